"""moe_forward_noalloc, the forward for callers that cannot allocate device
memory, against moe_forward on the same inputs: two calls in a row on one
device (the second with fewer tokens, so it runs on what the first left in the
library's scratch), every output equal bit for bit; shapes beyond the scratch
are refused before anything is launched."""
import pytest
import torch

from parity_helpers import log, shape_of
from sparse_mixture_experts_23_amd import _lib as L
from sparse_mixture_experts_23_amd import api
from sparse_mixture_experts_23_amd.workloads import MoEConfig, MoEInputs, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(shape, inp):
    T, k, E, d = shape.T, shape.k, shape.E, shape.d
    out = dict(y=torch.full((T, d), float("nan"), device=DEV),
               topk_ids=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
               topk_w=torch.full((T, k), float("nan"), device=DEV),
               load=torch.full((E,), -7, dtype=torch.int32, device=DEV),
               slot=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
               stats=torch.full((L.MOE_STAT_COUNT,), -7, dtype=torch.int32, device=DEV),
               status=torch.full((1,), -7, dtype=torch.int32, device=DEV))
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    rc = L.moe_forward_noalloc(shape, p(inp.x), p(inp.w_r), p(inp.b_r), p(inp.w_gate), p(inp.w_up), p(inp.w_down),
                               p(inp.s_gate), p(inp.s_up), p(inp.s_down), p(out["y"]), p(out["topk_ids"]),
                               p(out["topk_w"]), p(out["load"]), p(out["slot"]), p(out["stats"]), p(out["status"]),
                               torch.cuda.current_stream().cuda_stream)
    L.check(rc, "moe_forward_noalloc")
    return out


CASES = [
    # E <= 8 router (16-token workgroups, counts for the dispatch), shared expert, capacity drops
    (MoEConfig("noalloc_e8_shared", T=300, d=512, m=256, E=8, k=2, dtype="bf16", gate_mode=0, cf=(5, 4),
               bias="zipf", m_shared=128, cfg_id=70), 41),
    # the one-workgroup front of small batches, then a smaller one
    (MoEConfig("noalloc_front", T=12, d=1024, m=512, E=8, k=2, dtype="bf16", gate_mode=1, cf=None, m_shared=256,
               cfg_id=71), 5),
    # E > 64 (score GEMM + selection), several rounds of GEMM tiles
    (MoEConfig("noalloc_many", T=1500, d=512, m=384, E=100, k=6, dtype="bf16", gate_mode=0, cf=(5, 4),
               bias="zipf", cfg_id=72), 333),
    # fp32 layer
    (MoEConfig("noalloc_f32", T=200, d=96, m=64, E=6, k=2, dtype="f32", gate_mode=0, cf=(1, 1), cfg_id=73), 17),
    # fp32 over several token blocks: the grouped-row copy with the placement inside it
    (MoEConfig("noalloc_f32_copy", T=600, d=128, m=64, E=12, k=3, dtype="f32", gate_mode=0, cf=(1, 2),
               cfg_id=74), 300),
]


@pytest.mark.parametrize("cfg,T2", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_equals_forward_on_two_calls(cfg, T2):
    inp = make_inputs(cfg, 0, DEV)
    for T in (cfg.T, T2):   # the second call is smaller and reuses the scratch the first left behind
        c = cfg.with_tokens(T)
        sub = MoEInputs(**{**inp.__dict__, "cfg": c, "x": inp.x[:T].contiguous()})
        shape = shape_of(c)
        ref = api.forward(shape, sub.x, sub.w_r, sub.b_r, sub.w_gate, sub.w_up, sub.w_down, sub.s_gate, sub.s_up,
                          sub.s_down)
        got = _noalloc(shape, sub)
        torch.cuda.synchronize()
        assert int(got["status"].item()) == L.MOE_OK
        for name in ("y", "topk_ids", "topk_w", "load", "slot", "stats", "status"):
            assert torch.equal(got[name], getattr(ref, name)), f"{cfg.name} T={T}: {name} differs"
        log(f"[noalloc] {cfg.name} T={T}: equal to moe_forward")


def test_noalloc_refuses_shapes_beyond_the_scratch():
    big = api.make_shape(4096, 4096, 14336, 8, 2, 0, L.MOE_GATE_RENORM, torch.bfloat16)
    assert L.moe_workspace_bytes(big, L.MOE_WS_FORWARD) > L.MOE_NOALLOC_SCRATCH_BYTES
    fake = 4096   # never dereferenced: the call returns before launching
    args = [fake] * 16
    rc = L.moe_forward_noalloc(big, *args, torch.cuda.current_stream().cuda_stream)
    assert rc == L.MOE_ERR_WORKSPACE_TOO_SMALL
    small = api.make_shape(512, 4096, 14336, 8, 2, 0, L.MOE_GATE_RENORM, torch.bfloat16)
    assert L.moe_workspace_bytes(small, L.MOE_WS_FORWARD) <= L.MOE_NOALLOC_SCRATCH_BYTES
