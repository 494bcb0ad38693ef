"""Streams and graphs, through the C ABI.

* One plan used from two non-default streams at once: every call only
  enqueues on the stream it is given, the plan is read-only, so the results
  equal those of the same calls made one after the other, bit for bit.
* HIP graph capture: the forward + JVP and the backward allocate nothing,
  never synchronise and record no memset, so one graph can hold both.  The
  graph is replayed several times, with eager work (new inputs, outputs
  overwritten) and synchronisations between the replays, and every replay is
  checked against eager calls on the same inputs, bit for bit.
"""
import pytest
import torch

import seeded_inputs as si
import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS
from gpu_util import small_workload, device_inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _inputs(w):
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    return x


class _Buffers:
    def __init__(self, plan, like):
        self.o, self.to, self.dq, self.dk, self.dv = (torch.empty_like(like) for _ in range(5))
        self.lse = torch.empty(like.shape[:3], dtype=torch.float32, device=like.device)
        self.ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device=like.device)

    def outputs(self):
        return (self.o, self.to, self.lse, self.dq, self.dk, self.dv)


def _call(plan, x, b, stream=None):
    aj.attn_jvp_fwd(plan, *(x[t] for t in TENSORS), b.o, b.to, b.lse, stream=stream)
    aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], b.o, b.lse, x["do"], b.dq, b.dk, b.dv, b.ws, stream=stream)


@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("fp32", 64)])
def test_one_plan_on_two_streams(dtype, d):
    wa = small_workload(700, 160, 9, 3, 1, heads=2, d=d, dtype=dtype)
    wb = small_workload(701, 160, 9, 3, 1, heads=2, d=d, dtype=dtype)
    xa, xb = _inputs(wa), _inputs(wb)
    plan = aj.attn_jvp_create(wa.desc, wa.batch, wa.heads, wa.head_dim,
                              aj.ATTN_JVP_BF16 if dtype == "bf16" else aj.ATTN_JVP_FP32)
    ra, rb = _Buffers(plan, xa["q"]), _Buffers(plan, xb["q"])
    _call(plan, xa, ra)
    _call(plan, xb, rb)
    torch.cuda.synchronize()
    ga, gb = _Buffers(plan, xa["q"]), _Buffers(plan, xb["q"])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):  # interleaved, so that the two streams' kernels overlap
        _call(plan, xa, ga, stream=s1)
        _call(plan, xb, gb, stream=s2)
    torch.cuda.synchronize()
    for ref, got in ((ra, ga), (rb, gb)):
        for a, b in zip(ref.outputs(), got.outputs()):
            assert torch.equal(_bits(a), _bits(b))


def test_graph_capture_and_replay():
    w = small_workload(710, 160, 9, 3, 1, heads=2)
    x = _inputs(w)
    plan = aj.attn_jvp_create(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    g_buf = _Buffers(plan, x["q"])
    # warm-up on a side stream (the library checks the device once, outside capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(plan, x, g_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(plan, x, g_buf)  # on the capture stream (torch's current stream inside the block)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(711)
    for replay in range(4):
        # eager work between replays: new inputs in the captured buffers, outputs overwritten
        for t in list(TENSORS) + ["do"]:
            x[t].copy_(torch.randn(x[t].shape, device="cuda", generator=gen) * (0.1 if t.startswith("t") else 1.0))
        for out in g_buf.outputs():
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = _Buffers(plan, x["q"])
        _call(plan, x, ref)
        torch.cuda.synchronize()
        for a, b in zip(ref.outputs(), g_buf.outputs()):
            assert torch.equal(_bits(a), _bits(b)), f"replay {replay}"
