"""GPU: the torch custom ops (route, dispatch, combine and their autograd)
against the oracle, eagerly, under HIP graph capture and under torch.compile.

The layer is route -> dispatch -> experts -> combine with a toy expert
Y = bf16(fp32(rows) * row_w * scale[row_expert]) (scale a power of two, so the
CPU and GPU give the same bits), and the loss sum(fp32(out) * G).  The
reference runs the oracle for every step the library takes and plain CPU
torch for the expert:

  forward:  out bit-exact;
  backward: grad_x bit-exact (the gradient rows it sums are elementwise, hence
            identical on CPU and GPU); grad_topk_w within
            |d| <= 1e-5 * sum_h |g_h * f_h| of the CPU value (the expert's
            row-weight gradient is a float sum whose order torch does not fix).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from combine_topk_idx_multihot_amd import ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.moe_device_check(0)
    yield


def say(msg):
    print(msg, flush=True)


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16)


class Case:
    # the default shape routes in 5 blocks with the local experts taking most
    # slots (k * EL >= 2E), so the route writes its row list and the dispatch
    # and the combine backward walk it, also under graph capture and compile
    def __init__(self, T=640, k=4, E=24, lb=4, EL=16, P=4, H=512, seed=0, sync_free=False,
                 empty=False):
        rng = np.random.default_rng(seed)
        self.T, self.k, self.E, self.lb, self.EL, self.P, self.H = T, k, E, lb, EL, P, H
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1, allow_dup=True)
        if empty:
            idx[:] = -1
        self.idx = idx.astype(np.int32)
        self.w = rng.random((T, k), dtype=np.float32)
        self.x = inputs.bf16_normal((T, H), rng)
        self.G = rng.standard_normal((T, H)).astype(np.float32)
        self.scale = np.float32(2.0) ** (np.arange(EL + 1) % 3 - 1).astype(np.float32)
        self.C = oracle.capacity_min(T, k, EL, P) + 37 if sync_free else 0

    def experts(self, scale):
        def f(rows, row_w, row_expert):
            return (rows.float() * row_w[:, None] * scale[row_expert.long()][:, None]).to(
                torch.bfloat16)
        return f

    def device_inputs(self):
        x = from_bits(self.x).cuda().requires_grad_(True)
        w = torch.from_numpy(self.w).cuda().requires_grad_(True)
        return (x, torch.from_numpy(self.idx).cuda(), w, torch.from_numpy(self.G).cuda(),
                torch.from_numpy(self.scale).cuda())

    def layer(self, x, idx, w, G, scale):
        out = ops.moe_layer(x, idx, w, self.experts(scale), self.E, self.lb, self.EL, self.P,
                            self.C)
        loss = (out.float() * G).sum()
        gx, gw = torch.autograd.grad(loss, (x, w))
        return out, gx, gw

    def reference(self):
        """The oracle for the library's steps, CPU torch for the expert."""
        sf = self.C > 0
        ref = oracle.route(self.idx, self.E, self.lb, self.EL, self.P, sync_free=sf, C=self.C,
                           w=self.w, x=self.x)
        assert ref.rc == oracle.OK
        rows = from_bits(ref.rows).requires_grad_(True)
        rw = torch.from_numpy(ref.row_w.copy()).requires_grad_(True)
        Y = self.experts(torch.from_numpy(self.scale))(rows, rw, torch.from_numpy(ref.row_expert))
        out = oracle.combine(self.idx, ref.row_of_slot, bits(Y), self.E, self.lb, self.EL)
        g_out = bits(torch.from_numpy(self.G).to(torch.bfloat16))
        grad_Y, _ = oracle.combine_bwd(self.idx, ref.row_of_slot, ref.row_token, g_out, self.E,
                                       self.lb, self.EL, R=ref.R)
        Y.backward(from_bits(grad_Y))
        gx, gw = oracle.dispatch_bwd(self.idx, ref.row_of_slot, bits(rows.grad), self.E, self.lb,
                                     self.EL, grad_row_w=rw.grad.numpy())
        # bound on each row-weight gradient's rounding: sum_h |dY_h * scale * rows_h|
        s = torch.from_numpy(self.scale)[torch.from_numpy(ref.row_expert).long()][:, None]
        mag = (from_bits(grad_Y).double() * s.double() * rows.detach().double()).abs().sum(1)
        ros = ref.row_of_slot
        bound = np.where(ros >= 0, mag.numpy()[np.clip(ros, 0, None)], 0.0) if ref.R else \
            np.zeros_like(self.w, dtype=np.float64)
        return out, gx, gw, bound, ref.R

    def check(self, out, gx, gw, ref, what):
        r_out, r_gx, r_gw, bound, _ = ref
        np.testing.assert_array_equal(bits(out), r_out, err_msg=f"{what}: out")
        np.testing.assert_array_equal(bits(gx), r_gx, err_msg=f"{what}: grad_x")
        d = np.abs(gw.detach().cpu().numpy().astype(np.float64) - r_gw.astype(np.float64))
        assert np.all(d <= 1e-5 * bound + 1e-30), f"{what}: grad_topk_w off by {d.max()}"


@pytest.mark.parametrize("sync_free", [False, True])
@pytest.mark.parametrize("empty", [False, True])
def test_layer_forward_backward_matches_oracle(sync_free, empty):
    c = Case(seed=11, sync_free=sync_free, empty=empty)
    say(f"ops layer sync_free={sync_free} empty={empty} T={c.T} k={c.k} E={c.E} EL={c.EL}")
    out, gx, gw = c.layer(*c.device_inputs())
    torch.cuda.synchronize()
    c.check(out, gx, gw, c.reference(), "eager")


def test_layer_int64_ids_and_full_local_range():
    c = Case(T=257, k=8, E=32, lb=0, EL=32, P=1, H=768, seed=5)
    say("ops layer int64 ids, EL=E")
    x, idx, w, G, scale = c.device_inputs()
    out, gx, gw = c.layer(x, idx.long(), w, G, scale)
    torch.cuda.synchronize()
    c.check(out, gx, gw, c.reference(), "int64")


def test_graph_capture_replays_match_oracle():
    """Sync-free forward and backward captured once, replayed on new inputs."""
    c = Case(seed=21, sync_free=True)
    say("ops graph capture: warm-up")
    x, idx, w, G, scale = c.device_inputs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            c.layer(x, idx, w, G, scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out, gx, gw = c.layer(x, idx, w, G, scale)
    for seed in (31, 32, 33):
        say(f"ops graph replay seed={seed}")
        n = Case(seed=seed, sync_free=True)
        with torch.no_grad():
            x.copy_(from_bits(n.x))
            idx.copy_(torch.from_numpy(n.idx))
            w.copy_(torch.from_numpy(n.w))
            G.copy_(torch.from_numpy(n.G))
        g.replay()
        torch.cuda.synchronize()
        n.check(out, gx, gw, n.reference(), f"replay {seed}")
        # eager work between replays
        e_out, _, _ = n.layer(*n.device_inputs())
        torch.cuda.synchronize()
        assert torch.equal(e_out, out)


def test_torch_compile_traces_the_ops():
    c = Case(seed=41, sync_free=True)
    say("ops torch.compile(aot_eager, fullgraph)")
    x, idx, w, G, scale = c.device_inputs()

    def forward(x, idx, w, scale):
        return ops.moe_layer(x, idx, w, c.experts(scale), c.E, c.lb, c.EL, c.P, c.C)

    # one graph, forward and backward compiled by AOTAutograd around the ops
    fn = torch.compile(forward, backend="aot_eager", fullgraph=True)
    out = fn(x, idx, w, scale)
    (out.float() * G).sum().backward()
    torch.cuda.synchronize()
    c.check(out, x.grad, w.grad, c.reference(), "compiled")


def test_opcheck():
    c = Case(T=64, k=4, E=16, lb=0, EL=16, P=2, H=256, seed=51, sync_free=True)
    say("ops opcheck")
    x, idx, w, _, _ = c.device_inputs()
    meta = ops.route(idx, c.E, c.lb, c.EL, c.P, c.C)
    torch.library.opcheck(ops.route, (idx, c.E, c.lb, c.EL, c.P, c.C))
    args = (x, w) + tuple(meta[:6]) + (c.E, c.lb, c.P, c.C, c.C)
    torch.library.opcheck(ops.dispatch, args)
    rows = ops.dispatch(*args)[0].detach().requires_grad_(True)
    torch.library.opcheck(ops.combine, (rows,) + tuple(meta[:6]) + (c.E, c.lb, c.P, c.C))


def test_fp8_dispatch_op_matches_oracle():
    c = Case(T=333, k=4, E=24, lb=4, EL=16, P=4, H=768, seed=61, sync_free=True)
    say("ops dispatch_fp8 (sync-free, H=768)")
    x, idx, w, _, _ = c.device_inputs()
    meta = ops.route(idx, c.E, c.lb, c.EL, c.P, c.C)
    q, s, rw, rt, re = ops.dispatch_fp8(x.detach(), w.detach(), *meta[:6], c.E, c.lb, c.P, c.C,
                                        c.C)
    torch.cuda.synchronize()
    ref = oracle.route(c.idx, c.E, c.lb, c.EL, c.P, sync_free=True, C=c.C, w=c.w)
    rq, rs = oracle.dispatch_fp8(c.x, ref.row_token)
    np.testing.assert_array_equal(q.view(torch.uint8).cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    np.testing.assert_array_equal(rt.cpu().numpy(), ref.row_token)
    np.testing.assert_array_equal(re.cpu().numpy(), ref.row_expert)
    args = (x.detach(), w.detach()) + tuple(meta[:6]) + (c.E, c.lb, c.P, c.C, c.C)
    torch.library.opcheck(ops.dispatch_fp8, args)
