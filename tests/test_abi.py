"""C-ABI contract of libgdr on the CPU: exports, status strings, validation.

Every call here fails validation (or is a zero-sized no-op), which the
library guarantees happens before any HIP call, so no device is touched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_08_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, NULL, SHAPE, UNSUP, MISAL, WS, ENUM, HIP, ALIAS, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.library_path()):
        from gated_delta_rule_08_amd import build
        build.build()
    return gdr.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdr_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_what_binding_lists():
    assert _declared_functions() == sorted(gdr.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gdr.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version(lib):
    text = open(HEADER).read()
    ver = int(re.search(r"#define GDR_ABI_VERSION (\d+)", text).group(1))
    assert gdr.gdr_abi_version() == ver


def test_status_strings(lib):
    for code, tag in [(OK, "GDR_OK"), (NULL, "NULL_PTR"), (SHAPE, "BAD_SHAPE"),
                      (UNSUP, "UNSUPPORTED"), (MISAL, "MISALIGNED"), (WS, "WORKSPACE"),
                      (ENUM, "BAD_ENUM"), (HIP, "GDR_ERR_HIP"), (ALIAS, "ALIAS"), (SCRATCH, "SCRATCH")]:
        assert tag in gdr.gdr_status_string(code)
    assert gdr.gdr_status_string(12345) == "unknown gdr status"


# Fake, non-NULL, 256-byte aligned "device" addresses: only ever passed to
# calls that are rejected by validation.
P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]


def decode(lib, gate=0, dtype=1, B=2, H=3, dk=128, dv=128, ptrs=None):
    p = list(P[:8]) if ptrs is None else ptrs
    return lib.gdr_decode_step(gate, dtype, B, H, dk, dv, 1.0, *p)


def prefill(lib, gate=0, dtype=1, B=2, T=70, H=3, dk=128, dv=128, chunk=64, ptrs=None,
            ws=None, ws_bytes=0):
    p = list(P[:8]) if ptrs is None else ptrs
    return lib.gdr_chunk_prefill(gate, dtype, B, T, H, dk, dv, chunk, 1.0, *p,
                                 ws, ws_bytes, None)


def test_decode_validation(lib):
    assert decode(lib, gate=2) == ENUM
    assert decode(lib, dtype=7) == ENUM
    assert decode(lib, B=-1) == SHAPE
    assert decode(lib, H=-5) == SHAPE
    assert decode(lib, dk=96) == UNSUP
    assert decode(lib, dv=8) == UNSUP
    assert decode(lib, B=1 << 30, H=1 << 10) == SHAPE
    for i in range(7):  # q k v alpha beta state o
        ptrs = list(P[:8])
        ptrs[i] = None
        assert decode(lib, ptrs=ptrs) == NULL, i
    for i in (0, 1, 2, 5, 6):  # q k v state o need 16-byte alignment
        ptrs = list(P[:8])
        ptrs[i] = ctypes.c_void_p(P[i].value + 8)
        assert decode(lib, ptrs=ptrs) == MISAL, i
    ptrs = list(P[:8])
    ptrs[3] = ctypes.c_void_p(P[3].value + 4)  # KDA alpha needs 16-byte alignment
    assert decode(lib, gate=1, ptrs=ptrs) == MISAL
    ptrs = list(P[:8])
    ptrs[4] = ctypes.c_void_p(P[4].value + 2)  # beta needs 4-byte alignment
    assert decode(lib, ptrs=ptrs) == MISAL


def multi(lib, gate=0, dtype=1, B=2, T=4, H=3, dk=128, dv=128, ptrs=None):
    # q k v alpha beta state o states; the states buffer (T x the state) is
    # placed far from the rest unless a case moves it
    p = list(P[:7]) + [ctypes.c_void_p(0x7000000)] if ptrs is None else ptrs
    return lib.gdr_decode_multi(gate, dtype, B, T, H, dk, dv, 1.0, *p, None)


def _mptrs():
    return list(P[:7]) + [ctypes.c_void_p(0x7000000)]


def test_decode_multi_validation(lib):
    assert multi(lib, gate=3) == ENUM
    assert multi(lib, dtype=-1) == ENUM
    assert multi(lib, T=-1) == SHAPE
    assert multi(lib, B=-2) == SHAPE
    assert multi(lib, T=65) == UNSUP  # a verify window, not a prompt
    assert multi(lib, dk=48) == UNSUP
    for i in range(7):  # q k v alpha beta state o (states may be NULL)
        ptrs = _mptrs()
        ptrs[i] = None
        assert multi(lib, ptrs=ptrs) == NULL, i
    ptrs = _mptrs()
    ptrs[7] = ctypes.c_void_p(0x7000000 + 8)  # states need 16-byte alignment
    assert multi(lib, ptrs=ptrs) == MISAL
    ptrs = _mptrs()
    ptrs[3] = ctypes.c_void_p(P[3].value + 4)  # KDA alpha needs 16-byte alignment
    assert multi(lib, gate=1, ptrs=ptrs) == MISAL
    la = 2 * 3 * 128 * 128 * 4  # bytes of the state
    base = 0x40000000
    ptrs = _mptrs()
    ptrs[5] = ctypes.c_void_p(base)
    ptrs[7] = ctypes.c_void_p(base + 1024)  # states start inside the state
    assert multi(lib, ptrs=ptrs) == ALIAS
    ptrs[7] = ctypes.c_void_p(base - 4 * la + 256)  # states end inside it
    assert multi(lib, ptrs=ptrs) == ALIAS


def test_decode_multi_empty_is_noop(lib):
    assert multi(lib, T=0, ptrs=[None] * 8) == OK
    assert multi(lib, B=0, ptrs=[None] * 8) == OK
    assert multi(lib, H=0, ptrs=[None] * 8) == OK


def test_decode_zero_size_is_noop(lib):
    assert decode(lib, B=0, ptrs=[None] * 8) == OK
    assert decode(lib, H=0, ptrs=[None] * 8) == OK


def test_prefill_validation(lib):
    assert prefill(lib, gate=-1) == ENUM
    assert prefill(lib, dtype=2) == ENUM
    assert prefill(lib, T=-1) == SHAPE
    assert prefill(lib, chunk=32) == UNSUP
    assert prefill(lib, dk=256) == UNSUP
    ptrs = list(P[:8])
    ptrs[6] = None  # state_out
    assert prefill(lib, ptrs=ptrs) == NULL
    for i in (0, 1, 2, 3, 4, 7):  # q k v alpha beta o
        ptrs = list(P[:8])
        ptrs[i] = None
        assert prefill(lib, ptrs=ptrs) == NULL, i
    ptrs = list(P[:8])
    ptrs[5] = ctypes.c_void_p(P[6].value + 64)  # state_in overlaps state_out partially
    assert prefill(lib, ptrs=ptrs) == ALIAS
    ptrs = list(P[:8])
    ptrs[2] = ctypes.c_void_p(P[2].value + 2)
    assert prefill(lib, ptrs=ptrs) == MISAL
    assert prefill(lib, B=0, ptrs=[None] * 8) == OK


def varlen(lib, gate=0, dtype=1, N=3, total_T=100, max_T=64, H=2, dk=64, dv=64, chunk=64,
           ptrs=None, n_slots=4, ws=None, ws_bytes=0):
    # q k v alpha beta cu slots has states o
    p = list(P[:10]) if ptrs is None else ptrs
    return lib.gdr_chunk_prefill_varlen(gate, dtype, N, total_T, max_T, H, dk, dv, chunk, 1.0,
                                        *p[:9], n_slots, p[9], ws, ws_bytes, None)


def test_prefill_varlen_validation(lib):
    # GDN bf16 runs the fused schedule by default: no workspace needed
    assert varlen(lib, gate=5) == ENUM
    assert varlen(lib, N=-1) == SHAPE
    assert varlen(lib, max_T=-1) == SHAPE
    assert varlen(lib, n_slots=-1) == SHAPE
    assert varlen(lib, chunk=16) == UNSUP
    assert varlen(lib, dv=24) == UNSUP
    for i in (0, 1, 2, 3, 4, 5, 6, 8, 9):  # every pointer but has_state is required
        ptrs = list(P[:10])
        ptrs[i] = None
        assert varlen(lib, ptrs=ptrs) == NULL, i
    ptrs = list(P[:10])
    ptrs[5] = ctypes.c_void_p(P[5].value + 2)  # cu_seqlens: 4-byte alignment
    assert varlen(lib, ptrs=ptrs) == MISAL
    ptrs = list(P[:10])
    ptrs[8] = ctypes.c_void_p(P[8].value + 4)  # states: 16-byte alignment
    assert varlen(lib, ptrs=ptrs) == MISAL
    assert varlen(lib, N=0, ptrs=[None] * 10) == OK
    import torch
    need = gdr.gdr_chunk_prefill_varlen_workspace_bytes("kda", torch.bfloat16, 3, 64, 2, 64, 64)
    assert need > 0
    assert varlen(lib, gate=1) == WS
    assert varlen(lib, gate=1, ws=ctypes.c_void_p(0x100000), ws_bytes=need - 1) == WS


def test_workspace(lib):
    import torch
    # GDN bf16 (default schedule) and every fp32 prefill keep their intermediates on chip
    assert lib.gdr_chunk_prefill_workspace_bytes(0, 1, 4, 8192, 32, 128, 128, 64) == 0
    assert lib.gdr_chunk_prefill_workspace_bytes(1, 0, 1, 256, 2, 128, 128, 64) == 0
    # KDA bf16 stages one image per (b, h, chunk) of a range of chunks; a range
    # keeps all heads' images within 136 MiB, its chunk count rounded down to
    # a multiple of 256 / gcd(256, B H) (every chunk-local workgroup of the
    # 256 takes the same number of chunks)
    n = gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 32768, 32, 128, 128)
    n1 = gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 64, 1, 128, 128)
    assert n1 > 0 and n1 % 1024 == 0
    rc = min(512, (136 << 20) // (32 * n1))
    assert n == 32 * (rc // 8 * 8) * n1
    assert gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 65, 1, 128, 128) == 2 * n1
    assert gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 0, 1, 128, 128) == 0
    # invalid arguments need nothing
    assert lib.gdr_chunk_prefill_workspace_bytes(1, 1, 1, 64, 1, 96, 128, 64) == 0
    # a missing or short workspace is rejected before any device work
    assert prefill(lib, gate=1) == WS
    assert prefill(lib, gate=1, ws=P[8], ws_bytes=1024) == WS
    # the schedule is an argument: GDN can run split; KDA runs split only
    SF, SS = gdr.SCHED_FUSED, gdr.SCHED_SPLIT
    wsx = lib.gdr_chunk_prefill_workspace_bytes_ex
    assert wsx(1, 1, SS, 1, 64, 1, 128, 128, 64) == n1
    assert wsx(1, 1, SF, 1, 64, 1, 128, 128, 64) == 0          # KDA fused: unsupported
    assert wsx(0, 1, SF, 1, 64, 1, 128, 128, 64) == 0
    # GDN's image holds only the chunk's small tiles and gate factors
    g1 = gdr.gdr_chunk_prefill_workspace_bytes("gdn", torch.bfloat16, 1, 64, 1, 128, 128, flags=SS)
    assert 0 < g1 < n1 // 3 and g1 % 16 == 0
    assert wsx(0, 1, SS | 2, 1, 64, 1, 128, 128, 64) == g1      # with the sigmoid prologue
    assert wsx(0, 1, SS | 1, 1, 64, 1, 128, 128, 64) == 0       # GDN split cannot normalise
    assert wsx(0, 1, SS | SF, 1, 64, 1, 128, 128, 64) == 0      # both schedules: invalid
    assert wsx(0, 0, SS, 1, 64, 1, 128, 128, 64) == 0           # fp32: one schedule
    assert lib.gdr_chunk_prefill_varlen_workspace_bytes_ex(1, 1, SS, 1, 64, 1, 128, 128, 64) == n1
    assert lib.gdr_chunk_prefill_varlen_workspace_bytes_ex(0, 1, SS, 1, 64, 1, 128, 128, 64) == g1


def test_schedule_flag_validation(lib):
    """The schedule bits of the prefill calls, checked before the device."""
    SF, SS = gdr.SCHED_FUSED, gdr.SCHED_SPLIT

    def pre(gate, dtype, flags, ws=None, ws_bytes=0):
        return lib.gdr_chunk_prefill_ex(gate, dtype, flags, 2, 70, 3, 128, 128, 64, 1.0,
                                        *([None] * 8), ws, ws_bytes, None)

    assert pre(0, 1, SF | SS) == ENUM
    assert pre(0, 1, 16) == ENUM
    assert pre(1, 1, SF) == UNSUP          # KDA has no fused schedule
    assert pre(0, 0, SF) == UNSUP          # fp32 has one schedule
    assert pre(1, 0, SS) == UNSUP
    assert pre(0, 1, SF) == NULL           # valid, inputs missing
    assert pre(0, 1, SS) == WS             # the split schedule needs its workspace
    need = lib.gdr_chunk_prefill_workspace_bytes_ex(0, 1, SS, 2, 70, 3, 128, 128, 64)
    assert pre(0, 1, SS, ws=P[9], ws_bytes=need) == NULL
    assert pre(1, 1, SS) == WS and pre(1, 1, 0) == WS
    # the decode calls take no schedule bits
    p = list(P[:8])
    assert lib.gdr_decode_step_ex(0, 1, SF, 2, 3, 128, 128, 1.0, *p) == ENUM
    assert lib.gdr_decode_multi_ex(0, 1, SS, 2, 3, 4, 128, 128, 1.0, *[P[i] for i in range(9)]) == ENUM
    assert lib.gdr_chunk_prefill_varlen_ex(1, 1, SF, 2, 100, 70, 3, 128, 128, 64, 1.0, *([None] * 9), 4,
                                           None, None, 0, None) == UNSUP


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 16)
    with pytest.raises(ValueError):
        gdr.gdr_decode_step("gdn", q, q, q, torch.zeros(1, 1), torch.zeros(1, 1),
                            torch.zeros(1, 1, 16, 16), torch.zeros(1, 1, 16))


def test_prologue_flag_validation(lib):
    """Unknown prologue bits are BAD_ENUM; the normalising prologue in a bf16
    schedule that does not form the chunk-local products itself is
    UNSUPPORTED; everything is checked before the device is touched."""
    p = list(P[:8])
    assert lib.gdr_decode_step_ex(0, 1, 4, 2, 3, 128, 128, 1.0, *p) == ENUM
    assert lib.gdr_decode_step_ex(0, 1, -1, 2, 3, 128, 128, 1.0, *p) == ENUM
    assert lib.gdr_decode_step_ex(0, 1, 3, 0, 3, 128, 128, 1.0, *([None] * 8)) == OK
    assert lib.gdr_decode_step_ex(0, 1, 3, 2, 3, 100, 128, 1.0, *p) == UNSUP

    def pre(gate, dtype, flags, T=70):
        return lib.gdr_chunk_prefill_ex(gate, dtype, flags, 2, T, 3, 128, 128, 64, 1.0,
                                        *([None] * 8), None, 0, None)

    assert pre(0, 1, 16) == ENUM
    SF, SS = gdr.SCHED_FUSED, gdr.SCHED_SPLIT
    # GDN normalises in the fused kernel, KDA in the split one
    assert pre(0, 1, 1 | SF) == NULL and pre(0, 1, 1 | SS) == UNSUP
    assert pre(1, 1, 1 | SS) == WS and pre(1, 1, 1 | SF) == UNSUP
    assert pre(0, 1, 2 | SF) == NULL and pre(0, 1, 2 | SS) == WS  # the sigmoid runs in every schedule
    assert pre(1, 0, 3) == NULL        # fp32 path: both
    assert pre(0, 1, 3) == NULL and pre(1, 1, 3) == WS


def test_backward_validation(lib):
    """Validation of gdr_chunk_backward before any device work."""
    nul = [None] * 14

    def bwd(gate=0, dtype=1, B=2, T=70, H=3, dk=128, dv=128, chunk=64, ptrs=None, ws=None, ws_bytes=0):
        p = nul if ptrs is None else ptrs
        return lib.gdr_chunk_backward(gate, dtype, B, T, H, dk, dv, chunk, 1.0, *p, ws, ws_bytes, None)

    assert bwd(gate=3) == ENUM
    assert bwd(dtype=7) == ENUM
    assert bwd(B=-1) == SHAPE
    assert bwd(dk=48) == UNSUP
    assert bwd(chunk=32) == UNSUP
    need = lib.gdr_chunk_backward_workspace_bytes(0, 1, 2, 70, 3, 128, 128, 64)
    assert need > 0
    assert lib.gdr_chunk_backward_workspace_bytes(0, 1, 2, 0, 3, 128, 128, 64) == 0
    assert bwd() == WS                                        # workspace missing
    ws = ctypes.c_void_p(0x40000000)
    assert bwd(ws=ws, ws_bytes=need) == NULL                  # inputs missing
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(14)]
    p[5] = None                                               # state_in may be NULL
    p[7] = None                                               # grad_state_out may be NULL
    p[13] = None                                              # grad_state_in may be NULL
    bad = list(p)
    bad[8] = ctypes.c_void_p(0x10008)                         # grad_q misaligned
    assert bwd(ptrs=bad, ws=ws, ws_bytes=need) == MISAL
    assert bwd(B=0, ptrs=nul) == OK                           # empty batch: no-op
    # one workgroup per (b, h, chunk): 2^22 of them would overflow the dispatch
    assert bwd(B=1, T=64 * (1 << 22), H=1, ptrs=p, ws=ws, ws_bytes=need) == SHAPE
    assert bwd(B=2, T=64 * (1 << 21), H=1, ptrs=p, ws=ws, ws_bytes=need) == SHAPE
    assert lib.gdr_chunk_backward_workspace_bytes(0, 1, 1, 64 * (1 << 22), 1, 128, 128, 64) == 0
    # the 16-column slice grids of the chains: 600,000 heads x 8 slices
    assert bwd(B=600000, T=64, H=1, ptrs=p, ws=ws, ws_bytes=1 << 62) == SHAPE
    # a workspace below the one-pass size runs in chunk ranges: the smallest
    # accepted is the one-chunk-range size
    rng = lib.gdr_chunk_backward_workspace_bytes_ranged
    rng.restype = ctypes.c_size_t
    one = rng(0, 1, 2, 70, 3, 128, 128, 64, 1)
    assert 0 < one < need
    assert rng(0, 1, 2, 70, 3, 128, 128, 64, 2) == need      # two chunks: the whole sequence
    assert rng(0, 1, 2, 70, 3, 128, 128, 64, 0) == 0         # invalid range
    assert rng(0, 1, 2, 70, 3, 96, 128, 64, 1) == 0          # invalid arguments
    assert bwd(ptrs=bad, ws=ws, ws_bytes=one) == MISAL        # accepted size, then pointer checks
    assert bwd(ptrs=bad, ws=ws, ws_bytes=one - 4) == WS
    T = 64 * 512
    full = lib.gdr_chunk_backward_workspace_bytes(1, 1, 1, T, 32, 128, 128, 64)
    r128 = rng(1, 1, 1, T, 32, 128, 128, 64, 128)
    assert r128 < full and r128 <= 2 * 10 ** 9                 # the KDA workload in 2 GB
    assert rng(0, 1, 4, 64 * 128, 32, 128, 128, 64, 32) <= 2 * 10 ** 9  # and the GDN one


def test_decode_grid_limit(lib):
    """A decode whose dispatch would exceed 2^32 work-items is a shape error,
    reported before any device call: 70 M heads of 16 x 16 (one wavefront each)."""
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(7)]
    assert lib.gdr_decode_step(0, 0, 70_000_000, 1, 16, 16, 1.0, *p, None) == SHAPE
    assert lib.gdr_decode_step(1, 1, 35_000_000, 2, 16, 16, 1.0, *p, None) == SHAPE


def test_prologue_ex_variants_validation(lib):
    """The verify and packed variable-length calls take the same flags."""
    p9 = [P[i] for i in range(9)]
    assert lib.gdr_decode_multi_ex(0, 1, 4, 2, 3, 4, 128, 128, 1.0, *p9) == ENUM
    assert lib.gdr_decode_multi_ex(0, 1, 3, 2, 65, 4, 128, 128, 1.0, *p9) == UNSUP
    assert lib.gdr_decode_multi_ex(0, 1, 3, 2, 0, 4, 128, 128, 1.0, *([None] * 9)) == OK

    def vl(flags, gate=0, dtype=1):
        return lib.gdr_chunk_prefill_varlen_ex(gate, dtype, flags, 2, 100, 70, 3, 128, 128, 64, 1.0,
                                               *([None] * 9), 4, None, None, 0, None)

    assert vl(16) == ENUM
    assert vl(1 | gdr.SCHED_SPLIT) == UNSUP            # GDN normalises only in the fused kernel
    assert vl(1 | gdr.SCHED_FUSED, gate=1) == UNSUP    # KDA has no fused schedule
    assert vl(3) == NULL and vl(3, dtype=0) == NULL


def test_noalloc_validation(lib):
    """gdr_chunk_prefill_noalloc: the checks of gdr_chunk_prefill_ex, no
    workspace, and a clear error where one chunk of every head would not fit
    its fixed 96 MiB scratch -- all before any device call."""
    def na(gate=1, dtype=1, flags=0, B=2, T=70, H=3, dk=128, dv=128, chunk=64, ptrs=None):
        p = list(P[:8]) if ptrs is None else ptrs
        return lib.gdr_chunk_prefill_noalloc(gate, dtype, flags, B, T, H, dk, dv, chunk, 1.0, *p, None)

    assert na(gate=2) == ENUM
    assert na(flags=gdr.SCHED_FUSED | gdr.SCHED_SPLIT) == ENUM
    assert na(flags=gdr.SCHED_FUSED) == UNSUP                 # KDA: split only
    assert na(chunk=32) == UNSUP
    assert na(B=-1) == SHAPE
    assert na(B=0, ptrs=[None] * 8) == OK
    ptrs = list(P[:8])
    ptrs[0] = None
    assert na(ptrs=ptrs) == NULL
    # 68 KiB images: 1445 heads fit the scratch, 1446 do not (KDA, dk = 128)
    img = gdr.gdr_chunk_prefill_workspace_bytes("kda", _torch().bfloat16, 1, 64, 1, 128, 128)
    assert 1445 * img <= (96 << 20) < 1446 * img
    assert na(B=1, H=1446) == SCRATCH
    assert na(B=2, H=723) == SCRATCH
    assert na(B=1, H=1446, T=0) != SCRATCH                    # T == 0 needs no scratch
    assert na(gate=0, B=1, H=1446) != SCRATCH                 # GDN fused needs none
    assert na(gate=0, flags=gdr.SCHED_SPLIT, B=1, H=1446) != SCRATCH  # the small GDN image fits


def _torch():
    import torch
    return torch
