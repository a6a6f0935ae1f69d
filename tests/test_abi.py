"""The C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments before any launch.  Runs without a GPU: every call here fails
validation (or has T == 0) and returns before touching the HIP runtime.

The calls pass fake device addresses.  With a GPU visible, a validation
regression would launch kernels on them, so this file refuses to run where a
device is visible (counting devices does not initialise the runtime)."""
import ctypes
import os
import re

import pytest
import torch

if torch.cuda.device_count() > 0:
    pytest.skip("fake-pointer validation tests run only where no GPU is visible", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")


@pytest.fixture(scope="module")
def lib():
    from transformer_depth_wise_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from transformer_depth_wise_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attnres_\w+)\s*\(", text, re.M)))


def test_header_declares_every_entry_point():
    names = declared_functions()
    for n in ("attnres_phase1", "attnres_phase1_first_prenorm", "attnres_phase1_workspace_bytes", "attnres_phase2_merge",
              "attnres_phase1_accumulate",
              "attnres_phase2_backward", "attnres_phase1_backward",
              "attnres_phase2_merge_multi", "attnres_full", "attnres_block_accumulate", "attnres_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_uses_the_same_names():
    import transformer_depth_wise_amd as tdw
    for name in declared_functions():
        if name != "attnres_status_string":
            assert callable(getattr(tdw, name)), name


A = 1 << 20  # a 16-byte aligned fake device address; never dereferenced here
# Every call below must fail validation or have T == 0: a call that passed
# validation with these fake pointers would launch a kernel on them.
EINVAL, EDTYPE, EALIGN, EALIAS = 1, 2, 3, 4


def p(x):
    return ctypes.c_void_p(x)


def checked(rc):
    # ATTNRES_EHIP here means validation let fake pointers through to a launch
    assert rc != 5, "validation passed fake pointers to a kernel launch"
    return rc


def phase1(lib, dt=1, sdt=None, src=A, n=3, stride=4096 * 64, T=4096, d=64, w=8 * A, kg=None, S=4, eps=1e-6,
           out=16 * A, m=None, lse=24 * A, ws=32 * A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attnres_phase1_workspace_bytes(T, d, n, S)
    sdt = dt if sdt is None else sdt
    return checked(lib.attnres_phase1(dt, sdt, p(src), n, stride, T, d, p(w), p(kg), S, eps, p(out), p(m), p(lse),
                                      p(ws), ws_bytes, None))


def test_phase1_validation(lib):
    assert phase1(lib, dt=7) == EDTYPE
    assert phase1(lib, sdt=7) == EDTYPE
    assert phase1(lib, dt=0, sdt=1) == EDTYPE     # bf16 sources, fp32 outputs: not a supported pair
    assert phase1(lib, dt=1, sdt=2) == EDTYPE     # P24 is a partial-sum format only
    assert phase1(lib, dt=1, sdt=0, n=17, S=1) == EINVAL   # fp32 sources with bf16 outputs: at most 16
    assert phase1(lib, dt=1, sdt=0, S=1, ws=None, ws_bytes=0) == EINVAL  # ... and a workspace even for S == 1
    assert phase1(lib, d=12) == EALIGN
    assert phase1(lib, d=0) == EINVAL
    assert phase1(lib, d=16392) == EINVAL
    assert phase1(lib, n=0) == EINVAL
    assert phase1(lib, S=0) == EINVAL
    assert phase1(lib, n=17) == EINVAL            # more than 16 sources with S >= 2
    assert phase1(lib, n=33, S=1) == EINVAL
    assert phase1(lib, src=None) == EINVAL
    assert phase1(lib, lse=None) == EINVAL
    assert phase1(lib, stride=100) == EINVAL      # slabs would overlap
    assert phase1(lib, stride=4096 * 64 + 4) == EALIGN
    assert phase1(lib, src=A + 4) == EALIGN
    assert phase1(lib, out=A + 4096 * 64) == EALIAS   # output inside the source slabs
    assert phase1(lib, lse=16 * A + 8) == EALIAS      # stats inside the output
    assert phase1(lib, lse=24 * A + 2) == EALIGN
    assert phase1(lib, eps=-1.0) == EINVAL
    assert phase1(lib, T=1 << 31) == EINVAL              # more than ATTNRES_MAX_T tokens
    assert phase1(lib, S=4097) == EINVAL                 # more than ATTNRES_MAX_QUERIES
    assert phase1(lib, n=1, stride=-8) == EINVAL         # strides are >= 0 even where unused
    assert phase1(lib, stride=(1 << 40) + 8) == EINVAL   # beyond ATTNRES_MAX_STRIDE
    assert lib.attnres_phase1_workspace_bytes(1 << 31, 64, 2, 4) == -1
    assert phase1(lib, ws=None) == EINVAL                # S >= 2 needs the workspace
    assert phase1(lib, ws_bytes=100) == EINVAL           # too small
    assert phase1(lib, ws=16 * A + 64) == EALIAS         # workspace inside the output
    # packed queries: 32 rows x 4 bytes per channel, d rounded up to 128
    assert lib.attnres_phase1_workspace_bytes(4096, 64, 3, 4) == 16384 + 4096 * 3 * 4 * 4
    assert lib.attnres_phase1_workspace_bytes(4096, 64, 3, 40) == 16384 + 4096 * 3 * 32 * 4
    assert lib.attnres_phase1_workspace_bytes(4096, 64, 3, 1) == 16384 + 4096 * 3 * 4
    assert lib.attnres_phase1_workspace_bytes(16384, 7168, 8, 24) == 56 * 16384 + 16384 * 8 * 24 * 4
    assert lib.attnres_phase1_workspace_bytes(10, 136, 2, 2) == 2 * 16384 + 10 * 2 * 2 * 4
    assert lib.attnres_phase1_workspace_bytes(4096, 64, 20, 1) == 0     # > 16 sources: fused path only
    assert lib.attnres_phase1_workspace_bytes(4096, 64, 20, 2) == -1
    assert lib.attnres_phase1_workspace_bytes(4096, 12, 3, 4) == -1
    assert phase1(lib, T=0) == 0                      # nothing to do, nothing launched
    assert phase1(lib, T=0, src=None, out=None, lse=None) == 0


def first_prenorm(lib, dt=1, src=A, n=3, stride=4096 * 64, T=4096, d=64, w=8 * A, kg=None, S=4, out=16 * A,
                  m=None, lse=24 * A, gm=None, x=40 * A, h=None, ws=32 * A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attnres_phase1_workspace_bytes(T, d, n, S)
    return checked(lib.attnres_phase1_first_prenorm(dt, p(src), n, stride, T, d, p(w), p(kg), S, 1e-6, p(out),
                                                    p(m), p(lse), p(gm), p(x), p(h), p(ws), ws_bytes, None))


def test_phase1_first_prenorm_validation(lib):
    assert first_prenorm(lib, x=None) == EINVAL               # x_out is the point of the call
    assert first_prenorm(lib, out=None) == EINVAL             # several sources need the outputs
    assert first_prenorm(lib, n=17) == EINVAL
    assert first_prenorm(lib, n=20, S=1) == EINVAL            # S == 1 still runs the streaming pair
    assert first_prenorm(lib, S=1, ws=None) == EINVAL         # ... which needs the workspace
    assert first_prenorm(lib, x=A + 64) == EALIAS             # x_out inside the sources
    assert first_prenorm(lib, h=16 * A + 64) == EALIAS        # h_out inside out
    assert first_prenorm(lib, x=16 * A) == EALIAS             # x_out is out's slab 0
    assert first_prenorm(lib, h=40 * A + 16) == EALIAS        # h_out overlaps x_out
    assert first_prenorm(lib, gm=40 * A) == EALIAS            # an output over the PreNorm gain
    assert first_prenorm(lib, x=40 * A + 4) == EALIGN
    assert first_prenorm(lib, gm=48 * A + 2) == EALIGN
    assert first_prenorm(lib, d=12) == EALIGN
    assert first_prenorm(lib, dt=9) == EDTYPE
    assert first_prenorm(lib, T=0) == 0
    assert first_prenorm(lib, T=0, x=None) == EINVAL


def p1acc(lib, dt=1, sdt=None, vdt=None, src=A, n=3, stride=4096 * 64, T=4096, d=64, w=8 * A, kg=None, S=4, pdt=3,
          pin=54 * A, v2=52 * A, v=50 * A, out=16 * A, m=None, lse=24 * A, gm=None, x=None, h=None, ws=32 * A,
          ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attnres_phase1_workspace_bytes(T, d, n, S)
    sdt = dt if sdt is None else sdt
    vdt = dt if vdt is None else vdt
    return checked(lib.attnres_phase1_accumulate(dt, sdt, p(src), n, stride, T, d, p(w), p(kg), S, 1e-6, pdt, p(pin),
                                                 vdt, p(v2), p(v), p(out), p(m), p(lse), p(gm), p(x), p(h), p(ws),
                                                 ws_bytes, None))


def test_phase1_accumulate_validation(lib):
    slab2 = A + 2 * 4096 * 64 * 2                      # byte address of source slab n-1 = 2
    assert p1acc(lib, n=1) == EINVAL                   # the newest source is a block sum: n_src >= 2
    assert p1acc(lib, n=17) == EINVAL
    assert p1acc(lib, v=None) == EINVAL                # the block's last output is required
    assert p1acc(lib, pdt=9) == EDTYPE
    assert p1acc(lib, dt=0, pdt=0, sdt=1) == EDTYPE    # bf16 sources, fp32 outputs
    assert p1acc(lib, vdt=0, pdt=0) == EDTYPE          # fp32 pieces summed into bf16 sources
    assert p1acc(lib, vdt=9) == EDTYPE
    assert p1acc(lib, dt=0, sdt=0, vdt=1, pdt=3, T=0) == 0   # fp32 sources and outputs, bf16 pieces
    assert p1acc(lib, sdt=0, x=40 * A) == EINVAL       # the PreNorm of query 0 needs equal types
    assert p1acc(lib, gm=48 * A) == EINVAL             # a PreNorm gain without x_out
    assert p1acc(lib, h=44 * A) == EINVAL              # h_out without x_out
    assert p1acc(lib, v=slab2) == EALIAS               # a piece over the slab being written
    assert p1acc(lib, pin=slab2 + 4096) == EALIAS
    assert p1acc(lib, v2=16 * A + 64) == EALIAS        # a piece inside an output
    assert p1acc(lib, pin=24 * A) == EALIAS            # ... inside the statistics
    assert p1acc(lib, v=50 * A + 2) == EALIGN
    assert p1acc(lib, out=slab2) == EALIAS             # an output over the sources (as attnres_phase1)
    assert p1acc(lib, x=40 * A, out=None) == EINVAL    # as attnres_phase1_first_prenorm
    assert p1acc(lib, ws=None) == EINVAL
    assert p1acc(lib, d=12) == EALIGN
    assert p1acc(lib, S=0) == EINVAL
    assert p1acc(lib, T=1 << 31) == EINVAL
    assert p1acc(lib, T=0) == 0
    assert p1acc(lib, T=0, v=None, src=None) == 0


def p2b(lib, dt=1, T=1024, d=64, o=A, lse=2 * A, pdt=0, pin=None, v2=None, v=3 * A, w=4 * A, kg=None, gm=None,
        prenorm=1, dx=5 * A, dp=6 * A, g=7 * A, c=8 * A, gh=9 * A, dw=10 * A, dk=None, dgm=None, ws=11 * A,
        ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attnres_phase2_backward_workspace_bytes(T, d)
    return checked(lib.attnres_phase2_backward(dt, T, d, p(o), p(lse), pdt, p(pin), p(v2), p(v), p(w), p(kg), p(gm),
                                               prenorm, 1e-6, p(dx), p(dp), p(g), p(c), p(gh), p(dw), p(dk), p(dgm),
                                               p(ws), ws_bytes, None))


def test_phase2_backward_validation(lib):
    assert p2b(lib, dt=5) == EDTYPE
    assert p2b(lib, pin=12 * A, pdt=9) == EDTYPE
    assert p2b(lib, d=12) == EALIGN
    assert p2b(lib, v=None, pin=12 * A) == EINVAL          # a partial input needs the previous output
    assert p2b(lib, v=None, v2=12 * A) == EINVAL
    assert p2b(lib, g=None) == EINVAL
    assert p2b(lib, dp=None) == EINVAL                     # a partial source needs its gradient buffer
    assert p2b(lib, lse=None) == EINVAL
    assert p2b(lib, ws=None) == EINVAL
    assert p2b(lib, ws_bytes=8) == EINVAL
    assert p2b(lib, g=A + 64) == EALIAS                    # G over the phase-1 output
    assert p2b(lib, dp=5 * A + 16) == EALIAS               # the partial gradient over dx
    assert p2b(lib, c=9 * A) == EALIAS                     # the two per-token outputs overlap
    assert p2b(lib, dw=11 * A) == EALIAS                   # dw inside the workspace
    assert p2b(lib, g=7 * A + 8) == EALIGN
    assert p2b(lib, c=8 * A + 2) == EALIGN
    assert p2b(lib, T=0) == 0
    assert p2b(lib, T=0, v=None, pin=12 * A) == EINVAL
    assert lib.attnres_phase2_backward_workspace_bytes(0, 64) == 0
    assert lib.attnres_phase2_backward_workspace_bytes(10, 12) == -1


def p1b(lib, dt=1, sdt=None, src=A, n=3, stride=1024 * 64, T=1024, d=64, w=8 * A, kg=None, S=4, g=16 * A, gstride=1024 * 64,
        c=None, gh=None, ds=24 * A, dstride=1024 * 64, dw=32 * A, dk=None, ws=40 * A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attnres_phase1_backward_workspace_bytes(T, d, n, S)
    sdt = dt if sdt is None else sdt
    return checked(lib.attnres_phase1_backward(dt, sdt, p(src), n, stride, T, d, p(w), p(kg), S, 1e-6, p(g), gstride,
                                               p(c),
                                               p(gh), p(ds), dstride, 1, p(dw), p(dk), p(ws), ws_bytes, None))


def test_phase1_backward_validation(lib):
    assert p1b(lib, dt=3) == EDTYPE
    assert p1b(lib, dt=0, sdt=1) == EDTYPE                 # bf16 sources with fp32 G: not a supported pair
    assert p1b(lib, sdt=2) == EDTYPE
    assert p1b(lib, sdt=0, n=17, S=1) == EINVAL            # fp32 sources, bf16 G: at most 16, one site too
    # fp32 sources are twice as long: the second slab reaches the gradients
    assert p1b(lib, sdt=0, n=2, stride=1024 * 64, ds=A + 1024 * 64 * 2 * 2) == EALIAS
    assert p1b(lib, d=12) == EALIGN
    assert p1b(lib, n=0) == EINVAL
    assert p1b(lib, n=17) == EINVAL
    assert p1b(lib, S=33) == EINVAL
    assert p1b(lib, c=48 * A) == EINVAL                    # a partial weight without its G.p
    assert p1b(lib, g=None) == EINVAL
    assert p1b(lib, ds=None) == EINVAL
    assert p1b(lib, dw=None) == EINVAL
    assert p1b(lib, stride=100) == EINVAL
    assert p1b(lib, gstride=100) == EINVAL
    assert p1b(lib, dstride=100) == EINVAL
    assert p1b(lib, gstride=1024 * 64 + 4) == EALIGN
    assert p1b(lib, ws=None) == EINVAL
    assert p1b(lib, ws_bytes=64) == EINVAL
    assert p1b(lib, ds=A + 64) == EALIAS                   # gradients over the sources
    assert p1b(lib, dw=16 * A + 64) == EALIAS              # dw over G
    assert p1b(lib, dk=32 * A + 64, kg=48 * A) == EALIAS   # the two weight gradients overlap
    assert p1b(lib, ws=24 * A + 64) == EALIAS
    assert p1b(lib, T=0) == 0
    assert p1b(lib, gstride=1 << 41) == EINVAL
    assert lib.attnres_phase1_backward_workspace_bytes(1 << 31, 64, 3, 4) == -1
    assert lib.attnres_phase2_backward_workspace_bytes(1 << 31, 64) == -1
    # coefficients T x (S rounded up to 8) x n, folded queries S x d, per-range sums (2048 waves over
    # d / 256 groups), the queries packed as matrix-core operands (4096 bytes per 32 channels)
    assert lib.attnres_phase1_backward_workspace_bytes(1024, 64, 3, 4) == \
        4 * (1024 * 8 * 3 + 4 * 64 + 2048 * 4 * 64) + 2 * 4096
    assert lib.attnres_phase1_backward_workspace_bytes(16384, 7168, 8, 24) == \
        4 * (16384 * 24 * 8 + 24 * 7168 + 74 * 24 * 7168) + 224 * 4096
    assert lib.attnres_phase1_backward_workspace_bytes(8, 1000, 3, 4) % 16 == 0   # 1000 channels: 32 k-steps
    assert lib.attnres_phase1_backward_workspace_bytes(10, 64, 3, 33) == -1


def merge(lib, dt=1, T=1024, d=64, o=A, lse=2 * A, pdt=0, pin=None, v2=None, v=None, podt=0, pout=None, w=3 * A,
          kg=None, gm=None, h=None, x=4 * A):
    return checked(lib.attnres_phase2_merge(dt, T, d, p(o), p(lse), pdt, p(pin), p(v2), p(v), podt, p(pout), p(w),
                                            p(kg), p(gm), 1e-6, p(h), p(x), None))


def test_merge_validation(lib):
    assert merge(lib, x=None) == EINVAL                    # no output at all
    assert merge(lib, pin=5 * A) == EINVAL                 # partial without the previous output
    assert merge(lib, pout=5 * A) == EINVAL
    assert merge(lib, v2=6 * A) == EINVAL                  # two-before-previous output without the previous
    assert merge(lib, v=6 * A, v2=7 * A, pin=5 * A, pout=5 * A, pdt=2, podt=2, x=6 * A + 64) == EALIAS
    assert merge(lib, v=6 * A, v2=7 * A + 8) == EALIGN     # every row pointer 16-byte aligned
    assert merge(lib, v=6 * A, v2=7 * A, x=7 * A + 1024 * 64) == EALIAS  # output over the end of v2
    assert merge(lib, T=0, v=6 * A, v2=7 * A, pin=5 * A, pout=5 * A, pdt=2, podt=2) == 0
    assert merge(lib, pdt=9) == EDTYPE
    assert merge(lib, d=20) == EALIGN
    assert merge(lib, x=A + 64) == EALIAS                  # output over the phase-1 input
    assert merge(lib, v=6 * A, pin=5 * A, pout=5 * A + 16) == EALIAS   # shifted in-place
    assert merge(lib, v=6 * A, pin=5 * A, pout=5 * A, pdt=1) == EALIAS  # in place needs one format
    assert merge(lib, v=6 * A, pin=5 * A, pout=5 * A, pdt=2, podt=0) == EALIAS
    assert merge(lib, T=0, v=6 * A, pin=5 * A, pout=5 * A, pdt=2, podt=2) == 0  # P24 in place
    assert merge(lib, v=6 * A, pin=5 * A, podt=1, pout=7 * A) == EDTYPE  # partial_out is F32 or P24
    assert merge(lib, dt=2) == EDTYPE                                  # P24 is not a row format
    assert merge(lib, dt=0, pdt=1, v=6 * A, pin=5 * A) == EDTYPE        # bf16 partial with fp32 rows
    # a P24 partial spans 3 bytes per element: the low-byte plane starts 1024 x 64 x 2 bytes in
    assert merge(lib, v=7 * A + 1024 * 64 * 2, pin=5 * A, pdt=2, pout=7 * A, podt=2) == EALIAS
    assert merge(lib, T=0, v=6 * A, pin=5 * A, pout=5 * A, pdt=3, podt=3) == 0  # Q16 in place
    assert merge(lib, v=6 * A, pin=5 * A, pout=5 * A, pdt=3, podt=2) == EALIAS  # Q16 into P24 in place
    # a Q16 partial ends with T row exponents behind its 1024 x 64 values:
    # an output starting there overlaps it
    assert merge(lib, v=6 * A, pin=5 * A, pdt=3, pout=7 * A, podt=3, x=7 * A + 1024 * 64 * 2) == EALIAS
    assert merge(lib, pdt=4, v=6 * A, pin=5 * A) == EDTYPE
    assert merge(lib, T=0) == 0
    assert merge(lib, T=-1) == EINVAL
    assert merge(lib, T=1 << 31) == EINVAL
    assert merge(lib, T=0, o=None, lse=None, x=None) == 0               # empty: pointers unused


def test_full_and_accumulate_validation(lib):
    f = lambda **k: checked(lib.attnres_full(k.get("dt", 1), p(k.get("src", A)), k.get("n", 2), k.get("stride", 64 * 64),
                                     k.get("T", 64), k.get("d", 64), p(k.get("w", 2 * A)), None, None, 1e-6,
                                     p(k.get("h", 3 * A)), p(k.get("x")), p(k.get("lse")), None))
    assert f(n=0) == EINVAL
    assert f(n=33) == EINVAL
    assert f(h=None) == EINVAL
    assert f(h=A + 128) == EALIAS
    assert f(d=4) == EALIGN
    assert f(T=0) == 0
    assert f(T=1 << 40) == EINVAL
    assert f(stride=-64) == EINVAL
    acc = lambda **k: checked(lib.attnres_block_accumulate(k.get("dt", 1), k.get("T", 64), k.get("d", 64), k.get("pdt", 0),
                                                   p(k.get("pin")), p(k.get("v2")), p(k.get("v", A)),
                                                   p(k.get("out", 2 * A)), k.get("odt", k.get("dt", 1)),
                                                   None))
    assert acc(v=None) == EINVAL
    assert acc(odt=2) == EDTYPE                     # the block sum is dt or fp32
    assert acc(dt=0, odt=1) == EDTYPE               # fp32 rows summed into bf16: not a supported pair
    # an fp32 sum is twice as long as a bf16 row: ending where v starts as a
    # bf16 row would, it reaches into v
    assert acc(odt=0, out=A - 64 * 64 * 2) == EALIAS
    assert acc(out=A) == EALIAS
    assert acc(pin=2 * A, pdt=0) == EALIAS          # in place only with the same dtype
    assert acc(T=0, v=None, out=None) == 0
    assert acc(T=1 << 31, v=None, out=None) == EINVAL
    assert acc(dt=3) == EDTYPE
    assert acc(dt=2) == EDTYPE                      # P24 only for the partial
    assert acc(T=0, pin=5 * A, pdt=2) == 0
    assert acc(v2=2 * A + 64) == EALIAS             # out over v2
    assert acc(v2=3 * A + 4) == EALIGN
    assert acc(T=0, pin=5 * A, pdt=2, v2=3 * A) == 0


def test_merge_multi_validation(lib):
    mm = lambda **k: checked(lib.attnres_phase2_merge_multi(
        k.get("dt", 1), k.get("T", 64), k.get("d", 64), p(k.get("o", A)), p(k.get("lse", 2 * A)),
        p(k.get("src", 3 * A)), k.get("n", 2), k.get("stride", 64 * 64), p(k.get("w", 4 * A)), None, None, 1e-6,
        p(k.get("h")), p(k.get("x", 5 * A)), None))
    assert mm(n=17) == EINVAL                        # more than ATTNRES_MAX_GROUP_SOURCES
    assert mm(n=-1) == EINVAL
    assert mm(src=None) == EINVAL                    # sources announced but absent
    assert mm(w=None) == EINVAL
    assert mm(stride=64) == EINVAL                   # source slabs overlap
    assert mm(stride=64 * 64 + 4) == EALIGN
    assert mm(x=None) == EINVAL                      # no output
    assert mm(x=3 * A + 64 * 64 * 2) == EALIAS       # output over the second source
    assert mm(h=5 * A + 64) == EALIAS                # the two outputs overlap
    assert mm(dt=2) == EDTYPE
    assert mm(d=12) == EALIGN
    assert mm(T=0) == 0
    assert mm(stride=1 << 41) == EINVAL
    assert mm(T=0, n=0, src=None, w=None, o=None, lse=None, x=None) == 0


@pytest.mark.parametrize("entry", ["attnres_site_backward", "attnres_site_backward_accumulate"])
def test_site_backward_validation(lib, entry):
    acc = entry.endswith("accumulate")  # fp32 gradient rows
    sb = lambda **k: checked(getattr(lib, entry)(
        k.get("dt", 1), p(k.get("src", A)), k.get("n", 2), k.get("stride", 64 * 64), k.get("T", 64), k.get("d", 64),
        p(k.get("w", 2 * A)), None, None, k.get("prenorm", 1), 1e-6, p(k.get("dx", 3 * A)), p(k.get("dsrc", 4 * A)),
        k.get("dstride", 64 * 64), p(k.get("dw", 5 * A)), p(k.get("dkg")), p(k.get("dgm")), p(k.get("ws", 6 * A)),
        k.get("wsb", 1 << 20), None))
    assert lib.attnres_site_backward_workspace_bytes(64, 64) == 64 * 2 * 64 * 4   # one 64-thread team per token
    assert lib.attnres_site_backward_workspace_bytes(100000, 7168) == 1024 * 2 * 7168 * 4
    assert lib.attnres_site_backward_workspace_bytes(0, 64) == 0
    assert lib.attnres_site_backward_workspace_bytes(64, 12) == -1
    assert sb(n=0) == EINVAL
    assert sb(n=33) == EINVAL
    assert sb(wsb=16) == EINVAL                     # workspace too small
    assert sb(ws=None) == EINVAL
    assert sb(dw=None) == EINVAL
    assert sb(dstride=64) == EINVAL                 # gradient slabs overlap
    assert sb(dsrc=A + 64) == EALIAS                # gradient over the sources
    assert sb(dw=3 * A + 256) == EALIAS             # dw over dx
    assert sb(dkg=5 * A + 8) == EALIAS              # two [d] outputs overlap
    assert sb(ws=4 * A + 1024) == EALIAS            # workspace over the gradients
    if acc:
        # the fp32 gradient slabs end 2 * 4096 * 4 bytes after dsrc (bf16 ones: half that)
        assert sb(ws=4 * A + 20000) == EALIAS
    assert sb(stride=64 * 64 + 4) == EALIGN
    assert sb(dt=2) == EDTYPE
    assert sb(T=0, src=None, dx=None, dsrc=None, dw=None, ws=None) == 0
    assert sb(dstride=-64) == EINVAL
    assert lib.attnres_site_backward_workspace_bytes(1 << 31, 64) == -1


def test_status_strings(lib):
    from transformer_depth_wise_amd import _lib
    for code in range(6):
        assert _lib.status_string(code).startswith("ATTNRES_")


def test_stream_probe_validation(lib):
    def probe(nr=1, nw=1, src=A, dst=64 * A, nbytes=1 << 20, per_cu=2, unroll=2, nt=1):
        return checked(lib.attnres_stream_probe(nr, nw, p(src), p(dst), nbytes, per_cu, unroll, nt, None))
    assert probe(per_cu=0) == EINVAL
    assert probe(per_cu=17) == EINVAL
    assert probe(unroll=3) == EINVAL
    assert probe(nr=5) == EINVAL
    assert probe(nr=8, nw=1) == EINVAL     # the many-stream mixes are (8, 0), (9, 1) and (7, 24) only
    assert probe(nr=9, nw=0) == EINVAL
    assert probe(nr=7, nw=23) == EINVAL
    assert probe(nr=6, nw=24) == EINVAL
    assert probe(nr=10, nw=1) == EINVAL
    assert probe(nw=3) == EINVAL
    assert probe(nr=0, nw=0) == EINVAL
    assert probe(nbytes=0) == EINVAL
    assert probe(nbytes=(1 << 20) + 8) == EALIGN
    assert probe(src=None) == EINVAL
    assert probe(dst=None) == EINVAL
    assert probe(src=A + 4) == EALIGN
    assert probe(dst=A + (1 << 19)) == EALIAS           # written range overlaps the read one
    assert probe(nr=2, dst=A + (1 << 20)) == EALIAS     # second read stream overlaps the writes


def test_phase1_noalloc_validation(lib):
    # size checks return before the library looks up its scratch on a device
    def call(dt=1, n=3, T=4096, d=64, S=4, out=16 * A):
        return checked(lib.attnres_phase1_noalloc(dt, p(A), n, T * d, T, d, p(8 * A), None, S, 1e-6, p(out), None,
                                                  p(24 * A), None))
    ESCRATCH = 6
    assert call(dt=7) == EDTYPE
    assert call(n=17) == EINVAL                       # more than 16 sources with S >= 2
    assert call(d=12) == EALIGN
    assert call(T=200000, n=16, S=32) == ESCRATCH     # 410 MB of workspace > 64 MiB of scratch
    assert call(T=0) == 0                             # empty token set: nothing touched
    assert lib.attnres_phase1_workspace_bytes(16384, 7168, 16, 32) <= 64 << 20
    assert "ESCRATCH" in lib.attnres_status_string(ESCRATCH).decode()
