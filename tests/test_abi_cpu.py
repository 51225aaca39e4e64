"""CPU tests of the C ABI boundary: the library loads, exports every function
include/kda.h declares, and rejects bad arguments with the documented status
before touching the device. No kernel is launched here: every call below fails
validation (or, on a host without a GPU, the device check)."""
import ctypes
import re
from pathlib import Path

import pytest

from kda_gated_delta_chunk_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "kda.h"

A = 1 << 20  # a 16-byte aligned fake address; never dereferenced (validation fails first)


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_abi_version() == _lib.ABI_VERSION == 11


def test_status_strings():
    lib = _lib.load()
    for code, name in _lib.STATUS.items():
        assert lib.kda_status_string(code).decode() == name
    assert lib.kda_status_string(99).decode() == "KDA_ERROR_UNKNOWN"


def test_workspace_bytes():
    lib = _lib.load()
    def ws(*a, conv=0, operands=0):  # a kda_chunk_prep / kda_chunk_state pair
        return lib.kda_chunk_prep_workspace_bytes(*a, conv, operands)
    def wf(*a, conv=0, operands=0):  # one kda_chunk_fwd call
        return lib.kda_chunk_fwd_workspace_bytes(*a, conv, operands)
    n1 = ws(1, 4096, 96, 128, 128, 1, 16, 1)
    assert n1 > 0
    # grows with tokens and heads; bf16 blocks are smaller than fp32 blocks
    assert ws(1, 8192, 96, 128, 128, 1, 16, 1) > n1
    assert ws(1, 4096, 48, 128, 128, 1, 16, 1) < n1
    assert ws(1, 4096, 96, 128, 128, 1, 16, 0) > n1
    # packed batches need room for one extra partial chunk per sequence
    assert ws(1, 4096, 96, 128, 128, 16, 16, 1) > n1
    # 64-token chunks: one block of four 16-token sub-tiles per chunk
    n64 = ws(1, 4096, 96, 128, 128, 1, 64, 1)
    assert n64 > 0 and ws(1, 4096 + 64, 96, 128, 128, 1, 64, 1) > n64
    # unsupported sizes report 0
    for f in (ws, wf):
        assert f(1, 4096, 96, 96, 128, 1, 16, 1) == 0
        assert f(1, 4096, 96, 128, 128, 1, 32, 1) == 0
        assert f(2, 4096, 96, 128, 128, 3, 16, 1) == 0
        assert f(1, 4096, 0, 128, 128, 1, 16, 1) == 0
        assert f(1, 4096, 96, 128, 128, 1, 16, 1, conv=3) == 0
        assert f(1, 4096, 96, 128, 128, 1, 16, 1, operands=2) == 0
    # a convolution adds exactly the convolved v (B*T*H*V fp32 elements, or bf16 hi + lo parts), and where
    # the prep reads them convolved (fp32 I/O, 64-token chunks) the convolved q and k (fp32); the 16-token
    # bf16 prep convolves q and k as it reads them
    assert ws(1, 4096, 96, 128, 128, 1, 16, 1, conv=1) == n1 + 4096 * 96 * 128 * 4
    assert ws(1, 4096, 96, 128, 128, 1, 64, 1, conv=1) == n64 + 4096 * 96 * (128 + 2 * 128) * 4
    assert ws(1, 4096, 96, 64, 32, 1, 16, 0, conv=2) == ws(1, 4096, 96, 64, 32, 1, 16, 0) + 4096 * 96 * (32 + 2 * 64) * 4
    # fp16 operands: smaller factor blocks; only bf16 I/O at 16-token chunks without a convolution
    n16 = ws(1, 4096, 96, 128, 128, 1, 16, 1, operands=1)
    assert 0 < n16 < n1
    for f in (ws, wf):
        assert f(1, 4096, 96, 128, 128, 1, 16, 0, operands=1) == 0
        assert f(1, 4096, 96, 128, 128, 1, 64, 1, operands=1) == 0
        assert f(1, 4096, 96, 128, 128, 1, 16, 1, conv=1, operands=1) == 0
    # the least kda_chunk_fwd accepts: at 16-token chunks without a convolution the header and the chunk
    # table (the fused kernel), whatever the tokens; otherwise the two-pass size
    def wm(*a, conv=0, operands=0):
        return lib.kda_chunk_fwd_min_workspace_bytes(*a, conv, operands)
    for io in (0, 1):
        for o in ((0, 1) if io else (0,)):
            assert wm(1, 4096, 96, 128, 128, 1, 16, io, operands=o) == wm(1, 1 << 20, 96, 128, 128, 1, 16, io,
                                                                          operands=o) == 256 + 256 + 256
            assert wm(1, 4096, 96, 128, 128, 40, 16, io, operands=o) == 256 + 512 + 256
    assert wm(1, 4096, 96, 128, 128, 1, 64, 1) == n64
    assert wm(1, 4096, 96, 128, 128, 1, 16, 1, conv=1) == ws(1, 4096, 96, 128, 128, 1, 16, 1, conv=1)
    assert wm(1, 4096, 96, 128, 128, 1, 16, 1, operands=2) == 0 and wm(1, 4096, 96, 96, 128, 1, 16, 1) == 0
    # kda_chunk_fwd as two passes needs the split calls' workspace
    for a in [(1, 4096, 96, 128, 128, 1, 16, 1), (1, 4096, 96, 128, 128, 40, 16, 0), (1, 4096, 96, 128, 128, 1, 64, 1),
              (2, 300, 3, 64, 32, 2, 16, 1)]:
        for o in ((0, 1) if a[-1] == 1 and a[-2] == 16 else (0,)):
            assert wf(*a, operands=o) == ws(*a, operands=o) > 0
    assert wf(1, 4096, 96, 128, 128, 1, 16, 1, conv=1) == ws(1, 4096, 96, 128, 128, 1, 16, 1, conv=1)
    # the header (256 bytes) and the chunk table (num_seqs + 1 int64 and int32 entries, each 256-byte
    # aligned) come first: 39 more sequences add one partial chunk each and 256 bytes of table
    blk = ws(1, 64, 1, 32, 32, 2, 16, 1) - ws(1, 64, 1, 32, 32, 1, 16, 1)  # one more chunk, same table size
    assert ws(1, 64, 1, 32, 32, 40, 16, 1) - ws(1, 64, 1, 32, 32, 1, 16, 1) == 39 * blk + 256


def test_package_workspace_bytes_wrapper():
    """The package-level query passes every argument, with and without a convolution and per operand
    format, and agrees with the C query."""
    import kda_gated_delta_chunk_amd as kda
    lib = _lib.load()
    for conv in ("none", "short4", "short4_silu"):
        n = kda.workspace_bytes(1, 4096, 96, 128, 128, 1, 16, "bf16", conv=conv)
        assert n == lib.kda_chunk_fwd_workspace_bytes(1, 4096, 96, 128, 128, 1, 16, 1, _lib.CONVS[conv], 0) > 0
        assert kda.prep_workspace_bytes(1, 4096, 96, 128, 128, 1, 16, "bf16", conv=conv) >= n
    assert kda.workspace_bytes(1, 4096, 96, 128, 128, 1, 16, "bf16", conv="short4") > \
        kda.workspace_bytes(1, 4096, 96, 128, 128, 1, 16, "bf16")
    assert 0 < kda.prep_workspace_bytes(1, 64, 2, 32, 32, 1, 16, "bf16", operands="fp16") < \
        kda.prep_workspace_bytes(1, 64, 2, 32, 32, 1, 16, "bf16")
    assert kda.workspace_bytes(1, 64, 2, 32, 32, 1, 16, "fp32", operands="fp16") == 0
    with pytest.raises(ValueError):
        kda.workspace_bytes(1, 64, 2, 32, 32, 1, 16, "bf16", conv="long")
    with pytest.raises(ValueError):
        kda.workspace_bytes(1, 64, 2, 32, 32, 1, 16, "bf16", operands="fp8")


def test_workspace_status_rejects():
    lib = _lib.load()
    out = ctypes.c_int32(0)
    assert lib.kda_workspace_status(None, 1024, ctypes.byref(out), None) == INVALID
    assert lib.kda_workspace_status(A + 8, 1024, ctypes.byref(out), None) == INVALID
    assert lib.kda_workspace_status(A, 1024, None, None) == INVALID
    assert lib.kda_workspace_status(A, 255, ctypes.byref(out), None) == WS_SMALL


def _fwd(**kw):
    lib = _lib.load()
    a = dict(q=A, k=A, v=A, g=A, beta=A, og=None, S0=None, cu=None, B=1, T=64, H=2, K=32, V=32, N=1, chunk=16, io=1,
             gate=0, qkn=0, conv=0, cw=None, ops=0, odt=1, o=A, Sf=A, ws=A, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["og"], a["S0"], a["cu"], a["B"], a["T"],
                             a["H"],
                             a["K"], a["V"], a["N"], a["chunk"], a["io"], a["gate"], a["qkn"], a["conv"], a["cw"],
                             a["ops"], a["odt"], a["o"], a["Sf"], a["ws"],
                             a["wsb"], a["stream"])


def _prep(**kw):
    lib = _lib.load()
    a = dict(q=A, k=A, g=A, beta=A, cu=None, B=1, T=64, H=2, K=32, V=32, N=1, chunk=16, io=1, gate=0, qkn=0, conv=0,
             cw=None, ops=0, ws=A, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_prep(a["q"], a["k"], a["g"], a["beta"], a["cu"], a["B"], a["T"], a["H"], a["K"], a["V"],
                              a["N"], a["chunk"], a["io"], a["gate"], a["qkn"], a["conv"], a["cw"], a["ops"], a["ws"],
                              a["wsb"], a["stream"])


def _state(**kw):
    lib = _lib.load()
    a = dict(v=A, og=None, S0=None, cu=None, B=1, T=64, H=2, K=32, V=32, N=1, chunk=16, io=1, conv=0, cw=None, odt=1,
             o=A, Sf=A, ws=A, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_state(a["v"], a["og"], a["S0"], a["cu"], a["B"], a["T"], a["H"], a["K"], a["V"], a["N"],
                               a["chunk"], a["io"], a["conv"], a["cw"], a["odt"], a["o"], a["Sf"], a["ws"], a["wsb"],
                               a["stream"])


INVALID, UNSUP, WS_SMALL, NO_DEV = 1, 2, 3, 4


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=A + 8), INVALID),            # misaligned
    (dict(S0=A + 4), INVALID),
    (dict(og=A + 8), INVALID),           # o_gate misaligned
    (dict(cu=A + 2), INVALID),
    (dict(beta=A + 1), INVALID),         # bf16 beta needs 2-byte alignment
    (dict(beta=A + 2, io=0, odt=0), INVALID),  # fp32 beta needs 4-byte alignment
    (dict(B=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(H=0), INVALID),
    (dict(N=2), INVALID),                # num_seqs != B without cu_seqlens
    (dict(B=2, N=2, cu=A), INVALID),     # cu_seqlens needs B == 1
    (dict(io=7), INVALID),
    (dict(odt=-1), INVALID),
    (dict(gate=2), INVALID),
    (dict(gate=-1), INVALID),
    (dict(qkn=2), INVALID),
    (dict(qkn=-1), INVALID),
    (dict(conv=3), INVALID),
    (dict(conv=1), INVALID),             # a convolution needs its taps
    (dict(conv=1, cw=A + 4), INVALID),   # taps misaligned
    (dict(S0=A, Sf=A), INVALID),         # S0 aliases S_final
    (dict(T=1 << 40, H=96), INVALID),    # size overflow
    (dict(K=48), UNSUP),
    (dict(V=256), UNSUP),
    (dict(chunk=8), UNSUP),
    (dict(chunk=32), UNSUP),
    (dict(wsb=10), WS_SMALL),
    (dict(ws=None), WS_SMALL),
    (dict(ops=2), INVALID),              # unknown operand format
    (dict(ops=-1), INVALID),
    (dict(ops=1, io=0, odt=0), UNSUP),   # fp16 operands: bf16 I/O only
    (dict(ops=1, chunk=64), UNSUP),      # ... at 16-token chunks
    (dict(ops=1, conv=1, cw=A), UNSUP),  # ... without a convolution
    (dict(wsb=767), WS_SMALL),           # below the header and chunk table of the fused form
    (dict(wsb=10, chunk=64), WS_SMALL),  # 64-token chunks have no fused form
])
def test_chunk_fwd_rejects(kw, expect):
    assert _fwd(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID),
    (dict(ops=3), INVALID),
    (dict(ops=1, chunk=64), UNSUP),
    (dict(ops=1, io=0), UNSUP),
    (dict(K=48), UNSUP),
    (dict(wsb=100), WS_SMALL),
])
def test_chunk_prep_rejects(kw, expect):
    assert _prep(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(v=None), INVALID),
    (dict(o=None), INVALID),
    (dict(S0=A, Sf=A), INVALID),
    (dict(V=96), UNSUP),
    (dict(wsb=100), WS_SMALL),
])
def test_chunk_state_rejects(kw, expect):
    assert _state(**kw) == expect


def test_chunk_state_checks_the_smaller_layout_on_the_host():
    """kda_chunk_state takes the operand format from the header on the device; on the host it can only
    hold the workspace to the smaller of the two layouts (the fp16 one), and the kernels to the recorded
    one. A workspace below the fp16 size is refused before any launch."""
    lib = _lib.load()
    n16 = lib.kda_chunk_prep_workspace_bytes(1, 64, 2, 32, 32, 1, 16, 1, 0, 1)
    nbf = lib.kda_chunk_prep_workspace_bytes(1, 64, 2, 32, 32, 1, 16, 1, 0, 0)
    assert 0 < n16 < nbf
    assert _state(wsb=n16 - 1, cu=A + 4096) == WS_SMALL  # packed: the query's bound is exact


def _dec(**kw):
    lib = _lib.load()
    a = dict(q=A, k=A, v=A, g=A, beta=A, og=None, S=A + 4096, o=A + 8192, N=4, H=2, K=32, V=32, io=1, gate=0, qkn=0,
             conv=0, cw=None, cache=None, odt=1, stream=None)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["og"], a["S"], a["o"], a["N"], a["H"],
                               a["K"],
                               a["V"], a["io"], a["gate"], a["qkn"], a["conv"], a["cw"], a["cache"], a["odt"],
                               a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(S=None), INVALID),
    (dict(beta=None), INVALID),
    (dict(v=A + 2), INVALID),
    (dict(S=A), INVALID),                 # S aliases q
    (dict(og=A + 4096), INVALID),         # S aliases o_gate
    (dict(og=A + 2), INVALID),            # o_gate misaligned
    (dict(N=-1), INVALID),
    (dict(H=0), INVALID),
    (dict(io=3), INVALID),
    (dict(gate=5), INVALID),
    (dict(qkn=3), INVALID),
    (dict(conv=2, cw=A + 16384), INVALID),                # a convolution needs its cache
    (dict(conv=2, cw=A + 16384, cache=A + 4096), INVALID),  # cache aliases S
    (dict(conv=2, cw=A + 16384, cache=A + 20482), INVALID),  # cache misaligned
    (dict(K=16), UNSUP),
    (dict(V=96), UNSUP),
])
def test_decode_rejects(kw, expect):
    assert _dec(**kw) == expect


def test_decode_empty_batch_is_a_no_op():
    assert _dec(N=0, q=None, S=None) == 0


def _fwd_no_alloc(**kw):
    lib = _lib.load()
    a = dict(q=A, k=A, v=A, g=A, beta=A, og=None, S0=None, cu=None, B=1, T=64, H=2, K=32, V=32, N=1, chunk=16, io=1,
             gate=0, qkn=0, conv=0, cw=None, ops=0, odt=1, o=A, Sf=A, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_no_alloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["og"], a["S0"], a["cu"], a["B"],
                                      a["T"], a["H"], a["K"], a["V"], a["N"], a["chunk"], a["io"], a["gate"], a["qkn"],
                                      a["conv"], a["cw"], a["ops"], a["odt"], a["o"], a["Sf"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID),
    (dict(o=A + 8), INVALID),
    (dict(K=48), UNSUP),
    (dict(chunk=64, ops=1), UNSUP),
    (dict(S0=A + 4096, Sf=A + 4096), INVALID),
    # the least workspace over the scratch's 16 MiB: a convolution keeps the convolved q, k, v (4096 x 8 heads)
    (dict(T=4096, H=8, K=128, V=128, conv=2, cw=A), WS_SMALL),
    # ... or the chunk table of 2M packed sequences
    (dict(T=1 << 21, H=1, N=1 << 21, cu=A), WS_SMALL),
])
def test_no_alloc_rejects(kw, expect):
    assert _fwd_no_alloc(**kw) == expect


def test_no_alloc_scratch_limits():
    # what kda_chunk_fwd_no_alloc accepts is what fits in its scratch under kda_chunk_fwd's least workspace
    lib = _lib.load()
    least = lib.kda_chunk_fwd_min_workspace_bytes
    assert least(1, 4096, 8, 128, 128, 1, 16, 1, 2, 0) > _lib.NO_ALLOC_SCRATCH_BYTES
    assert least(1, 1 << 21, 1, 32, 32, 1 << 21, 16, 1, 0, 0) > _lib.NO_ALLOC_SCRATCH_BYTES
    assert least(1, 1 << 20, 96, 128, 128, 1, 16, 1, 0, 0) <= _lib.NO_ALLOC_SCRATCH_BYTES  # 1M tokens, fused


def _bwd(**kw):
    lib = _lib.load()
    a = dict(q=A, k=A + 4096, v=A + 8192, g=A + 12288, beta=A + 16384, og=None, S0=None, cu=None, do=A + 20480,
             dSf=None, dog=A + 7 * 65536 + 4096,
             B=1, T=64, H=2, K=32, V=32, N=1, io=1, gate=0, qk=0, conv=0, cw=None, dq=A + 65536, dk=A + 2 * 65536,
             dv=A + 3 * 65536, dg=A + 4 * 65536, db=A + 5 * 65536, dcw=None, dS0=A + 6 * 65536, ws=A + 8 * 65536,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["og"], a["S0"], a["cu"], a["do"], a["dSf"],
                             a["B"], a["T"], a["H"], a["K"], a["V"], a["N"], a["io"], a["gate"], a["qk"], a["conv"],
                             a["cw"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dog"], a["dcw"], a["dS0"], a["ws"],
                             a["wsb"], a["stream"])


CW, DCW = A + 9 * 65536, A + 10 * 65536  # conv taps and their gradient (fake addresses)


@pytest.mark.parametrize("kw,expect", [
    (dict(do=None), INVALID),
    (dict(dg=None), INVALID),
    (dict(q=A + 8), INVALID),             # misaligned
    (dict(dSf=A + 4), INVALID),
    (dict(beta=A + 16385), INVALID),      # bf16 beta needs 2-byte alignment
    (dict(cu=A + 2), INVALID),
    (dict(dq=A), INVALID),                # an output aliases an input
    (dict(dS0=A + 65536), INVALID),       # two outputs alias
    (dict(B=2, N=2, cu=A + 7 * 65536), INVALID),
    (dict(N=3), INVALID),
    (dict(io=4), INVALID),
    (dict(gate=2), INVALID),
    (dict(og=A + 7 * 65536 + 8192, dog=None), INVALID),   # an output gate needs its gradient
    (dict(og=A + 7 * 65536 + 8192, dog=A), INVALID),      # dL/dz aliases q
    (dict(og=A + 7 * 65536 + 8200), INVALID),             # o_gate misaligned
    (dict(H=0), INVALID),
    (dict(T=1 << 28, H=128), INVALID),   # the per-(chunk, head) grids would not be launchable
    (dict(K=48), UNSUP),
    (dict(V=256), UNSUP),
    (dict(wsb=100), WS_SMALL),
    (dict(ws=None), WS_SMALL),
    (dict(qk=2), INVALID),
    (dict(conv=3, cw=CW, dcw=DCW), INVALID),
    (dict(conv=1, cw=None, dcw=DCW), INVALID),            # a convolution needs its taps
    (dict(conv=1, cw=CW, dcw=None), INVALID),             # ... and their gradient
    (dict(conv=2, cw=CW, dcw=None, T=0), INVALID),        # also when there are no tokens
    (dict(conv=1, cw=CW + 4, dcw=DCW), INVALID),          # taps misaligned
    (dict(conv=1, cw=CW, dcw=DCW + 8), INVALID),          # gradient misaligned
    (dict(conv=1, cw=CW, dcw=CW), INVALID),               # the gradient aliases the taps
    (dict(conv=1, cw=CW, dcw=A + 65536), INVALID),        # ... or dq
])
def test_chunk_bwd_rejects(kw, expect):
    assert _bwd(**kw) == expect


def test_bwd_workspace_bytes():
    lib = _lib.load()
    ws = lib.kda_chunk_bwd_workspace_bytes
    # per (16-token chunk, head): a factor block (four 16 x K operand arrays, seven 16 x 16 ones and K decays,
    # rounded up to 64 floats) and X, W, dW (16 x V each); per pair of chunks of a sequence and head, one state
    # and one state gradient (K x V each; at most (chunks + sequences + 1) / 2 pairs); per token and head:
    # do * sigmoid(z) (V floats, used with an output gate)
    B, T, H, K, V = 2, 64, 3, 32, 64
    nc = B * (T // 16)
    fac = -(-(4 * 16 * K + 7 * 16 * 16 + K) // 64) * 64
    pairs = (nc + B + 1) // 2
    need = nc * H * (fac + 3 * 16 * V) * 4 + pairs * H * 2 * K * V * 4 + B * T * H * V * 4
    assert need <= ws(B, T, H, K, V, B, 0, 0) <= need + 10 * 256
    assert ws(1, 4096, 96, 128, 128, 16, 0, 0) > ws(1, 4096, 96, 128, 128, 1, 0, 0)  # one more chunk per sequence
    assert ws(1, 64, 2, 48, 32, 1, 0, 0) == 0 and ws(2, 64, 2, 32, 32, 1, 0, 0) == 0
    assert ws(B, T, H, K, V, B, 2, 0) == 0 and ws(B, T, H, K, V, B, 0, 3) == 0


def test_bwd_workspace_bytes_with_prologue():
    # the prologue adds its fp32 outputs and gradients (q, k; v with a convolution), the norm factors and the
    # taps' per-64-token partial sums
    ws = _lib.load().kda_chunk_bwd_workspace_bytes
    B, T, H, K, V = 2, 64, 3, 32, 64
    base = ws(B, T, H, K, V, B, 0, 0)
    n = B * T * H
    qk = 4 * n * K * 4
    norm = 2 * n * 4
    conv = 2 * n * V * 4 + -(-B * T // 64) * H * (2 * K + V) * 4 * 4
    for qc, cc, extra in ((1, 0, qk + norm), (0, 1, qk + conv), (0, 2, qk + conv), (1, 2, qk + norm + conv)):
        got = ws(B, T, H, K, V, B, qc, cc) - base
        assert extra <= got <= extra + 8 * 256, (qc, cc, got, extra)


def test_bwd_segmented_workspace_bytes():
    # segments of L tokens: one call's workspace for L tokens in L / 16 chunks of at most max(1, L / 64)
    # sequences, the states entering the segments of one sequence (ceil(T / L) - 1 of K x V per head), two state
    # gradients and the calls' sequence starts
    lib = _lib.load()
    seg, one = lib.kda_chunk_bwd_segmented_workspace_bytes, lib.kda_chunk_bwd_workspace_bytes
    B, T, H, K, V = 1, 4096, 4, 64, 64
    hkv = H * K * V * 4
    fac = -(-(4 * 16 * K + 7 * 16 * 16 + K) // 64) * 64
    for L in (32, 256, 1024):
        cap, nc = max(1, L // 64), L // 16
        core = nc * H * (fac + 3 * 16 * V) * 4 + (nc + cap + 1) // 2 * H * 2 * K * V * 4 + L * H * V * 4
        extra = (-(-T // L) - 1) * hkv + 2 * hkv
        slack = 16 * 256 + nc * 32 + 4 * (cap + 1) * 8
        got = seg(B, T, H, K, V, 1, 0, 0, L)
        assert core + extra <= got <= core + extra + slack, (L, got, core + extra)
    assert seg(B, T, H, K, V, 1, 0, 0, 256) < one(B, T, H, K, V, 1, 0, 0) / 4
    assert seg(B, T, H, K, V, 1, 1, 0, 64) > seg(B, T, H, K, V, 1, 0, 0, 64)  # the normalisation's buffers
    for L in (0, 16, 48, -32):
        assert seg(B, T, H, K, V, 1, 0, 0, L) == 0, L                      # not a positive multiple of 32
    assert seg(B, T, H, K, V, 1, 0, 1, 64) == 0 and seg(B, T, H, K, V, 1, 0, 2, 64) == 0  # no convolution
    assert seg(B, T, H, 48, V, 1, 0, 0, 64) == 0


def test_chunk_bwd_segmented_workspace_limits():
    lib = _lib.load()
    # below the least segmented workspace (32-token segments) the call reports a small workspace, and with a
    # convolution anything below one call's workspace
    least = min(lib.kda_chunk_bwd_segmented_workspace_bytes(1, 64, 2, 32, 32, 1, 0, 0, L) for L in (32, 64))
    assert _bwd(wsb=least - 1) == WS_SMALL
    full_conv = lib.kda_chunk_bwd_workspace_bytes(1, 64, 2, 32, 32, 1, 0, 1)
    assert _bwd(conv=1, cw=CW, dcw=DCW, wsb=full_conv // 2) == WS_SMALL


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="valid arguments would launch kernels on fake pointers")
def test_valid_arguments_without_a_device_report_no_device():
    assert _fwd() == NO_DEV
    assert _fwd(ops=1) == NO_DEV
    assert _fwd(wsb=768) == NO_DEV  # the fused form's workspace
    assert _prep() == NO_DEV
    assert _state() == NO_DEV
    assert _dec() == NO_DEV
    assert _bwd() == NO_DEV
    assert _bwd(wsb=_lib.load().kda_chunk_bwd_segmented_workspace_bytes(1, 64, 2, 32, 32, 1, 0, 0, 32)) == NO_DEV
    assert _fwd_no_alloc() == NO_DEV
    assert _fwd_no_alloc(T=1 << 20, H=96, K=128, V=128) == NO_DEV  # fits in the scratch as the fused kernel
    assert _bwd(qk=1, conv=2, cw=CW, dcw=DCW) == NO_DEV
    out = ctypes.c_int32(0)
    assert _lib.load().kda_workspace_status(A, 1024, ctypes.byref(out), None) == NO_DEV
