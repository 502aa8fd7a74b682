"""The two bf16 prefill schedules of GDN (fused; chunk-local kernel + chain
kernel), chosen by the GDR_SCHED_* flag, each match the oracle; they round
differently (the chain kernel applies the block inverse (I + A)^{-1} formed by
the chunk-local kernel, the fused one substitutes block by block), so they are
compared to the oracle, not to each other bit for bit.  KDA has the split
schedule only, which the same cases cover."""
from dataclasses import replace

import pytest
import torch

import gated_delta_rule_08_amd as gdr
import synth
from gpu_util import announce, ensure_built
from test_gpu_prefill import check, run_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


SCHED = {"fused": gdr.SCHED_FUSED, "split": gdr.SCHED_SPLIT}
PATHS = [("gdn", "fused"), ("gdn", "split"), ("kda", "split")]


def _run(path, gate, inp, scale=1.0):
    return run_prefill(gate, "bf16", inp, scale, flags=SCHED[path])


@pytest.mark.parametrize("gate,path", PATHS)
@pytest.mark.parametrize("T,dk,dv", [(1, 128, 128), (64, 128, 128), (130, 128, 128),
                                     (200, 16, 16), (150, 32, 64), (150, 64, 32),
                                     (100, 128, 16), (100, 16, 128)])
def test_paths_against_oracle(gate, path, T, dk, dv):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate, dtype="bf16",
                dk=dk, dv=dv)
    announce("prefill %s %s T=%d dk=%d dv=%d" % (path, gate, T, dk, dv))
    check(gate, "bf16", synth.make_inputs(w, B=2, T=T, H=3, seed=300 + T + dk), scale=0.8,
          flags=SCHED[path])


def test_paths_agree_long():
    """1000 tokens (16 chunks): both GDN schedules against the oracle and each other."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate="gdn", dtype="bf16")
    inp = synth.make_inputs(w, B=1, T=1000, H=3, seed=77)
    announce("prefill paths gdn T=1000")
    o_f, s_f = _run("fused", "gdn", inp)
    o_s, s_s = _run("split", "gdn", inp)
    scale_o = float(o_f.float().abs().max())
    scale_s = float(s_f.float().abs().max())
    assert float((o_f.float() - o_s.float()).abs().max()) <= 2e-2 * scale_o
    assert float((s_f - s_s).abs().max()) <= 2e-2 * scale_s
    check("gdn", "bf16", inp, flags=gdr.SCHED_SPLIT)


@pytest.mark.parametrize("gate,path", PATHS)
def test_each_path_against_oracle(gate, path):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate, dtype="bf16")
    announce("prefill %s %s vs oracle" % (gate, path))
    check(gate, "bf16", synth.make_inputs(w, B=2, T=333, H=5, seed=41), scale=0.6, flags=SCHED[path])


def test_split_gdn_full_size_every_head():
    """The GDN B=4 T=8192 H=32 d=128 workload through the split schedule,
    every head against one full oracle run."""
    w = synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128"]
    announce("prefill gdn full size, split schedule")
    check("gdn", "bf16", synth.make_inputs(w), flags=gdr.SCHED_SPLIT)


def test_split_workspace_passed_explicitly():
    """A caller-provided workspace (reused over two calls of different sizes)."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], dtype="bf16")
    big = synth.make_inputs(w, B=1, T=400, H=4, seed=5)
    small = synth.make_inputs(w, B=1, T=70, H=2, seed=6)
    need = gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 400, 4, 128, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    announce("prefill kda split, explicit workspace")
    for inp in (big, small):
        ref_o, ref_s = run_prefill("kda", "bf16", inp)
        d = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
        q, k, v = (d[x].to(torch.bfloat16) for x in ("q", "k", "v"))
        B, T, H, dk = q.shape
        o = torch.empty(B, T, H, v.shape[-1], device="cuda", dtype=torch.bfloat16)
        s = torch.empty(B, H, dk, v.shape[-1], device="cuda")
        gdr.gdr_chunk_prefill("kda", q, k, v, d["alpha"].float(), d["beta"].float(),
                              d["s0"].float(), s, o, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


def test_auto_workspace_on_a_side_stream():
    """workspace=None with the launch on another stream: the binding records
    its block on that stream, so blocks allocated and written on the current
    stream right after the call cannot be the one the kernels still use."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], dtype="bf16")
    inp = synth.make_inputs(w, B=1, T=3000, H=8, seed=15)
    ref_o, ref_s = run_prefill("kda", "bf16", inp)
    d = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
    q, k, v = (d[x].to(torch.bfloat16) for x in ("q", "k", "v"))
    a, b, s0 = d["alpha"].float(), d["beta"].float(), d["s0"].float()
    o = torch.empty_like(ref_o)
    s = torch.empty_like(ref_s)
    need = gdr.gdr_chunk_prefill_workspace_bytes("kda", torch.bfloat16, 1, 3000, 8, 128, 128)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    announce("prefill kda split, auto workspace on a side stream")
    gdr.gdr_chunk_prefill("kda", q, k, v, a, b, s0, s, o, stream=side)
    junk = [torch.full((need,), 255, dtype=torch.uint8, device="cuda") for _ in range(3)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
