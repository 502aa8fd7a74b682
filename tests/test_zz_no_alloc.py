"""gdr_chunk_prefill_noalloc (no workspace: the library's fixed device
scratch) called through the C ABI, against gdr_chunk_prefill_ex with a
workspace: the same kernels and arithmetic, so the outputs and final states
are bitwise equal.  Two calls in a row, the second smaller (the scratch keeps
the first call's images), for each schedule that uses the scratch and one
that does not."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_08_amd as gdr
import synth
from gpu_util import announce, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dev(inp):
    return {key: (None if val is None else torch.from_numpy(val).to(
        torch.bfloat16 if key in ("q", "k", "v") else torch.float32).cuda()) for key, val in inp.items()}


def _noalloc(gate, flags, d, s_out, o):
    lib = gdr.load_library()
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.gdr_chunk_prefill_noalloc(gdr.GATES[gate], 1, flags, B, T, H, dk, dv, 64, 0.9, ptr(d["q"]),
                                       ptr(d["k"]), ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]),
                                       ptr(d["s0"]), ptr(s_out), ptr(o),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, gdr.gdr_status_string(st)


@pytest.mark.parametrize("gate,flags", [("kda", 0), ("gdn", gdr.SCHED_SPLIT), ("gdn", 0)])
def test_noalloc_matches_the_workspace_call(gate, flags):
    w = synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128" if gate == "kda" else "gdn_prefill_b4_t8192_h32_d128"]
    # 256 heads: five chunks of all heads per 96 MiB range for KDA, so the
    # first call runs several ranges; the second call is small
    cases = [synth.make_inputs(w, B=4, T=1000, H=64, seed=21, s0="normal"),
             synth.make_inputs(w, B=1, T=130, H=3, seed=22, s0="normal")]
    for i, inp in enumerate(cases):
        d = _dev(inp)
        B, T, H, dk = d["q"].shape
        dv = d["v"].shape[-1]
        o_ref = torch.empty(B, T, H, dv, device="cuda", dtype=torch.bfloat16)
        s_ref = torch.empty(B, H, dk, dv, device="cuda")
        need = gdr.gdr_chunk_prefill_workspace_bytes(gate, torch.bfloat16, B, T, H, dk, dv, flags=flags)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        announce("prefill noalloc %s flags=%d call %d (B=%d T=%d H=%d)" % (gate, flags, i, B, T, H))
        gdr.gdr_chunk_prefill_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], s_ref, o_ref,
                                 flags=flags, scale=0.9, workspace=ws)
        o = torch.full_like(o_ref, 3.0)
        s = torch.full_like(s_ref, 3.0)
        _noalloc(gate, flags, d, s, o)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "o differs (call %d)" % i
        assert torch.equal(s, s_ref), "state differs (call %d)" % i
