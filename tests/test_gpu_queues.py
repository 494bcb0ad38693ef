"""The bf16 kernels' work queues (take_task in csrc/kernel_common.h; the ring
of queue slots in csrc/attn_jvp_api.hip).

Each call takes the next of 256 slots of per-XCD queue counters, its grid
holds half again as many workgroups as tasks, and the last workgroup to take
a task zeroes the slot again.  If a slot were left non-zero, or a position were
handed out twice or not at all, a later call would skip or repeat query or
key blocks.  So: more calls than there are slots (every slot is used at least
twice), alternating plans whose grids have fewer tasks than XCDs, one task
per XCD and many, forward + JVP, the forward without tangents, the backward
and the clean-tangent-zero forward (whose two kernels each use one slot one
after the other) and range-list plans; every output prefilled with NaN and
every call's bits equal to the first call's.  Then calls that overlap on two
streams, and replays of a captured HIP graph (whose launches keep the slot
they took at capture) between eager calls.
"""
import pytest
import torch

import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS
from gpu_util import log, small_workload, device_inputs

pytestmark = pytest.mark.gpu

N_SLOTS = 256  # kQueueSlots


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


class _Case:
    """One plan and its inputs; fwd() and bwd() return fresh NaN-prefilled outputs."""

    def __init__(self, w, ranges=False, ctz=False):
        self.w = w
        self.x = device_inputs(w)
        if ranges:
            n_tok, groups = w.mask_ranges()
            self.plan = aj.attn_jvp_create_ranges(n_tok, groups, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
            self.table = torch.from_numpy(aj.attn_jvp_plan_table(self.plan)).cuda()
        else:
            flags = aj.ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO if ctz else 0
            self.plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16, 0.0, flags)
            self.table = None
        self.n_tasks = w.batch * w.heads * self.plan.info["n_query_blocks"]
        self.d_o = torch.randn_like(self.x["q"], dtype=torch.float32).to(torch.bfloat16)
        self.o, _, self.lse = self.fwd()
        self.ws = torch.empty(aj.attn_jvp_bwd_workspace_size(self.plan) // 4, dtype=torch.float32, device="cuda")

    def _nan(self, like, dtype=None):
        return torch.full_like(like, float("nan"), dtype=dtype)

    def fwd(self):
        x = self.x
        o, to = self._nan(x["q"]), self._nan(x["q"])
        lse = torch.full(self.w.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        if self.table is None:
            aj.attn_jvp_fwd(self.plan, *(x[t] for t in TENSORS), o, to, lse)
        else:
            aj.attn_jvp_fwd_table(self.plan, self.table, *(x[t] for t in TENSORS), o, to, lse)
        return o, to, lse

    def prim(self):
        x = self.x
        o = self._nan(x["q"])
        lse = torch.full(self.w.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        if self.table is None:
            aj.attn_jvp_fwd_primal(self.plan, x["q"], x["k"], x["v"], o, lse)
        else:
            aj.attn_jvp_fwd_primal_table(self.plan, self.table, x["q"], x["k"], x["v"], o, lse)
        return o, lse

    def bwd(self):
        x = self.x
        dq, dk, dv = (self._nan(x["q"]) for _ in range(3))
        args = (x["q"], x["k"], x["v"], self.o, self.lse, self.d_o, dq, dk, dv, self.ws)
        if self.table is None:
            aj.attn_jvp_bwd(self.plan, *args)
        else:
            aj.attn_jvp_bwd_table(self.plan, self.table, *args)
        return dq, dk, dv


def test_queue_slots_are_reused_and_every_call_is_complete():
    cases = [
        _Case(small_workload(401, 50, 3, 1, 0, heads=1)),            # 2 tasks: six queues empty
        _Case(small_workload(402, 50, 5, 1, 1, heads=2)),            # 8 tasks: one per XCD
        _Case(small_workload(403, 37, 30, 2, 1, heads=3, batch=2)),  # 108 tasks
        _Case(small_workload(404, 40, 6, 3, 1, heads=2), ranges=True),
        _Case(small_workload(405, 50, 5, 1, 1, heads=1), ctz=True),   # 2 + 2 tasks in two launches
        _Case(small_workload(410, 37, 30, 2, 1, heads=3, batch=2), ctz=True),
    ]
    for c in cases:
        log(f"[queues] {c.w.name} desc={c.w.desc} B={c.w.batch} H={c.w.heads} tasks={c.n_tasks} "
            f"ranges={c.table is not None}")
    ref = [(c.fwd(), c.prim(), c.bwd()) for c in cases]
    torch.cuda.synchronize()
    for (f, pr, b) in ref:
        for t in f + pr + b:
            assert not torch.isnan(t).any(), "a block was never computed"
    calls = 0
    it = 0
    while calls < 2 * N_SLOTS + 16:
        for c, (rf, rp, rb) in zip(cases, ref):
            f = c.fwd()
            pr = c.prim()
            b = c.bwd()
            calls += 3
            for got, want in zip(f + pr + b, rf + rp + rb):
                if not torch.equal(_bits(got), _bits(want)):
                    torch.cuda.synchronize()
                    raise AssertionError(f"call {calls} ({c.w.name}): outputs differ from the first call's")
        it += 1
    torch.cuda.synchronize()
    log(f"    {calls} calls over {it} rounds, every one bit-identical to the first")


def test_calls_on_two_streams_at_once_take_different_slots():
    """Calls issued alternately on two streams overlap on the GPU; consecutive
    calls take consecutive slots, so each finds its own slot zeroed."""
    a = _Case(small_workload(406, 50, 5, 1, 1, heads=2))
    b = _Case(small_workload(407, 37, 30, 2, 1, heads=3, batch=2))
    log(f"[queues] two streams: {a.n_tasks} and {b.n_tasks} tasks")
    ref = {id(a): (a.fwd(), a.bwd()), id(b): (b.fwd(), b.bwd())}
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(60):
        for c, s in ((a, s1), (b, s2)):
            with torch.cuda.stream(s):
                outs.append((c, c.fwd(), c.bwd()))
    torch.cuda.synchronize()
    for i, (c, f, bw) in enumerate(outs):
        rf, rb = ref[id(c)]
        for got, want in zip(f + bw, rf + rb):
            assert torch.equal(_bits(got), _bits(want)), f"call {i} ({c.w.name}) differs"
    log(f"    {2 * len(outs)} calls on two streams, every one bit-identical to the first")


def test_graph_replays_find_their_queue_slot_zeroed():
    """A captured call keeps the queue slot it took at capture time; every
    replay finds it zeroed again (the last workgroup of the previous launch
    zeroed it), with eager calls of another plan between the replays.  The
    capture holds the forward and the no-allocation backward; outputs are
    prefilled with NaN before each replay."""
    c = _Case(small_workload(408, 40, 6, 3, 1, heads=2))
    other = _Case(small_workload(409, 50, 5, 1, 1, heads=1))
    x = c.x
    o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
    lse = torch.empty(c.w.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))

    def call():
        aj.attn_jvp_fwd(c.plan, *(x[t] for t in TENSORS), o, to, lse)
        aj.attn_jvp_bwd_noalloc(c.plan, x["q"], x["k"], x["v"], o, lse, c.d_o, dq, dk, dv)

    def nan_fill():
        for t in (o, to, lse, dq, dk, dv):
            t.fill_(float("nan"))

    nan_fill()
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, to, lse, dq, dk, dv)]
    for t in ref:
        assert not torch.isnan(t).any()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call on the capture stream before capturing
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(4):
        nan_fill()
        g.replay()
        for _ in range(3):
            other.fwd()
            other.bwd()
        torch.cuda.synchronize()
        for got, want in zip((o, to, lse, dq, dk, dv), ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {r} differs from the eager call"
    log("    4 graph replays, each bit-identical to the eager call")


def test_graph_replays_of_the_two_launch_calls():
    """A captured clean-tangent-zero forward (two launches, one slot) and a
    forward without tangents, replayed between eager calls of other plans;
    every replay bit-identical to the eager calls."""
    c = _Case(small_workload(411, 40, 6, 3, 1, heads=2), ctz=True)
    other = _Case(small_workload(412, 50, 5, 1, 1, heads=1))
    x = c.x
    o, to, po = torch.empty_like(x["q"]), torch.empty_like(x["q"]), torch.empty_like(x["q"])
    lse, plse = (torch.empty(c.w.shape[:3], dtype=torch.float32, device="cuda") for _ in range(2))

    def call():
        aj.attn_jvp_fwd(c.plan, *(x[t] for t in TENSORS), o, to, lse)
        aj.attn_jvp_fwd_primal(c.plan, x["q"], x["k"], x["v"], po, plse)

    def nan_fill():
        for t in (o, to, po, lse, plse):
            t.fill_(float("nan"))

    nan_fill()
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, to, po, lse, plse)]
    for t in ref:
        assert not torch.isnan(t).any()
    assert torch.equal(_bits(ref[2]), _bits(ref[0])) and torch.equal(_bits(ref[4]), _bits(ref[3]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(4):
        nan_fill()
        g.replay()
        for _ in range(3):
            other.fwd()
            other.prim()
        torch.cuda.synchronize()
        for got, want in zip((o, to, po, lse, plse), ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {r} differs from the eager call"
    log("    4 graph replays of the clean-tangent-zero and primal calls, each bit-identical")
