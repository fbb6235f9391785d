"""The torch custom ops on the CPU: registration, fake implementations and the
autograd wiring, traced with fake tensors (nothing runs the library here)."""
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import ops

OPS = ("route", "dispatch", "dispatch_fp8", "dispatch_bwd", "combine", "combine_bwd")


def test_ops_are_registered():
    for name in OPS:
        op = getattr(torch.ops.moe_mi355x, name).default
        schema = str(op._schema)
        assert schema.startswith(f"moe_mi355x::{name}(")
        assert "!" not in schema  # no op mutates its inputs


def test_fake_shapes():
    T, k, E, EL, H, P = 96, 8, 64, 32, 1024, 4
    C = T * k + EL * (P - 1)
    with FakeTensorMode():
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        meta = ops.route(idx, E, 16, EL, P, C)
        desc = B.make_desc(T, k, E, 16, EL, P, B.MOE_SYNC_FREE, False, C)
        ws = B.moe_route_workspace_size(desc)
        assert [tuple(t.shape) for t in meta] == [(T, E), (EL,), (EL + 1,), (T, k), (4,), (ws,),
                                                  (4,)]
        assert meta[5].dtype == torch.uint8 and meta[6].device.type == "cpu"
        rows, row_w, rt, re = ops.dispatch(x, w, *meta[:6], E, 16, P, C, C)
        assert rows.shape == (C, H) and rows.dtype == torch.bfloat16
        assert row_w.shape == rt.shape == re.shape == (C,)
        assert row_w.dtype == torch.float32 and rt.dtype == re.dtype == torch.int32
        q, sc, qw, qt, qe = ops.dispatch_fp8(x, w, *meta[:6], E, 16, P, C, C)
        assert q.shape == (C, H) and q.dtype == torch.float8_e4m3fn
        assert sc.shape == (C, H // 128) and sc.dtype == torch.float32
        assert qw.shape == qt.shape == qe.shape == (C,)
        out = ops.combine(rows, *meta[:6], E, 16, P, C)
        assert out.shape == (T, H) and out.dtype == torch.bfloat16
        gr = ops.combine_bwd(out, C, *meta[:6], E, 16, P, C)
        assert gr.shape == (C, H)
        gx, gw = ops.dispatch_bwd(rows, row_w, *meta[:6], E, 16, P, C)
        assert gx.shape == (T, H) and gw.shape == (T, k) and gw.dtype == torch.float32


def test_backward_traces_to_the_library_backward_ops():
    T, k, E, H, P = 64, 4, 16, 512, 4
    C = T * k + E * (P - 1)

    def step(x, idx, w, G):
        x = x.detach().requires_grad_(True)
        w = w.detach().requires_grad_(True)

        def experts(rows, row_w, row_expert):
            return (rows.float() * row_w[:, None]).to(torch.bfloat16)

        out = ops.moe_layer(x, idx, w, experts, E, pad_multiple=P, capacity=C)
        gx, gw = torch.autograd.grad((out.float() * G).sum(), (x, w))
        return out, gx, gw

    g = make_fx(step, tracing_mode="fake")(torch.zeros((T, H), dtype=torch.bfloat16),
                                           torch.zeros((T, k), dtype=torch.int32),
                                           torch.zeros((T, k)), torch.zeros((T, H)))
    called = [n.target for n in g.graph.nodes if n.op == "call_function"]
    names = [str(t) for t in called if "moe_mi355x" in str(t)]
    assert names == ["moe_mi355x.route.default", "moe_mi355x.dispatch.default",
                     "moe_mi355x.combine.default", "moe_mi355x.combine_bwd.default",
                     "moe_mi355x.dispatch_bwd.default"]
    outs = [n for n in g.graph.nodes if n.op == "output"][0].args[0]
    assert [tuple(o.meta["val"].shape) for o in outs] == [(T, H), (T, H), (T, k)]
