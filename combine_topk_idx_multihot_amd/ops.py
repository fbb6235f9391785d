"""torch.library custom ops over the C ABI: fake implementations and autograd.

"Add the deepep expert-parallel implementation", sections "Custom ops" and
"Training": dispatch and combine are custom ops with fake implementations and
registered autograd; the dispatch handle cannot cross an op boundary as an
object, so its tensors do and each op rebuilds it; gradients reach the tokens
and the routing weights.

Ops (namespace ``moe_mi355x``), each a thin marshal into the binding; every
step runs in the HIP library:

  route(topk_idx, num_experts, local_begin, num_local, pad_multiple, capacity)
      -> (routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
          workspace, host_status)
      capacity == 0 is the eager mode: host_status (CPU int32[4]) holds
      {total, flags, data rows, 0}, so R = host_status[0] with no further sync.
      capacity > 0 is the sync-free mode: R = capacity and nothing leaves the
      device (capturable; host_status stays zero).
  dispatch(x, topk_w, <handle tensors>, num_experts, local_begin, pad_multiple,
           capacity, R) -> (rows, row_w, row_token, row_expert)
      backward: dispatch_bwd (moe_dispatch_bwd) -> (grad_x, grad_topk_w)
  dispatch_fp8(same arguments as dispatch)
      -> (rows_q [R,H] float8_e4m3fn, row_scale [R,H/128], row_w, row_token,
          row_expert); E4M3 codes with one fp32 scale per 128 elements, no
      autograd (the codes are a quantization)
  combine(Y, <handle tensors>, num_experts, local_begin, pad_multiple,
          capacity) -> out [T,H] bf16
      backward: combine_bwd (moe_combine_bwd, the cached dispatch of grad_out)

<handle tensors> = routing_map, tokens_per_expert, padded_offsets, row_of_slot,
status, workspace, in that order.  The workspace carries the route's row list
(for dense routing), which the dispatch and the combine backward walk instead
of the tokens.  The handle fields the ops need but do not carry (T, k, the
number of local experts) are read off the tensors' shapes.

``moe_layer`` strings the ops together around a caller-supplied expert.
"""
from __future__ import annotations

import torch

from . import binding as B

_NS = "moe_mi355x"
_NO_HOST = torch.zeros(4, dtype=torch.int32)  # host status of handles that never route


def _desc(T, k, E, lb, EL, P, capacity, idx_i64=False):
    mode = B.MOE_SYNC_FREE if capacity > 0 else B.MOE_EAGER
    return B.make_desc(T, k, E, lb, EL, P, mode, idx_i64, capacity)


def _rebuild(routing_map, tpe, off, ros, status, workspace, E, lb, P, capacity):
    """The dispatch handle from its tensors."""
    T, k = ros.shape
    desc = _desc(T, k, E, lb, tpe.numel(), P, capacity)
    h = B.Handle(desc=desc, routing_map=routing_map, tokens_per_expert=tpe, padded_offsets=off,
                 row_of_slot=ros, status=status, host_status=_NO_HOST, workspace=workspace)
    return desc, h


# ---------------------------------------------------------------------------
# route
# ---------------------------------------------------------------------------
@torch.library.custom_op(f"{_NS}::route", mutates_args=())
def route(topk_idx: torch.Tensor, num_experts: int, local_begin: int, num_local: int,
          pad_multiple: int, capacity: int
          ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor,
                     torch.Tensor, torch.Tensor]:
    T, k = topk_idx.shape
    desc = _desc(T, k, num_experts, local_begin, num_local, pad_multiple, capacity,
                 topk_idx.dtype == torch.int64)
    dev = topk_idx.device
    eager = capacity == 0
    h = B.Handle(
        desc=desc,
        routing_map=torch.empty((T, num_experts), dtype=torch.uint8, device=dev),
        tokens_per_expert=torch.empty(num_local, dtype=torch.int32, device=dev),
        padded_offsets=torch.empty(num_local + 1, dtype=torch.int32, device=dev),
        row_of_slot=torch.empty((T, k), dtype=torch.int32, device=dev),
        status=torch.empty(4, dtype=torch.int32, device=dev),
        # eager: pinned, so the route kernel writes the count straight to the host
        host_status=torch.zeros(4, dtype=torch.int32, pin_memory=eager),
        # zeroed: the route leaves some of its bytes unwritten (never read by
        # the kernels), and an op's outputs must not depend on stale memory
        workspace=torch.zeros(B.moe_route_workspace_size(desc), dtype=torch.uint8, device=dev))
    B.moe_route_build(desc, topk_idx.contiguous(), h)
    return (h.routing_map, h.tokens_per_expert, h.padded_offsets, h.row_of_slot, h.status,
            h.workspace, h.host_status)


@route.register_fake
def _(topk_idx, num_experts, local_begin, num_local, pad_multiple, capacity):
    T, k = topk_idx.shape
    dev = topk_idx.device
    desc = _desc(T, k, num_experts, local_begin, num_local, pad_multiple, capacity,
                 topk_idx.dtype == torch.int64)
    return (topk_idx.new_empty((T, num_experts), dtype=torch.uint8),
            topk_idx.new_empty(num_local, dtype=torch.int32),
            topk_idx.new_empty(num_local + 1, dtype=torch.int32),
            topk_idx.new_empty((T, k), dtype=torch.int32),
            topk_idx.new_empty(4, dtype=torch.int32),
            topk_idx.new_empty(B.moe_route_workspace_size(desc), dtype=torch.uint8),
            torch.empty(4, dtype=torch.int32, device="cpu") if dev.type != "cpu"
            else topk_idx.new_empty(4, dtype=torch.int32))


# ---------------------------------------------------------------------------
# dispatch, with autograd through moe_dispatch_bwd
# ---------------------------------------------------------------------------
@torch.library.custom_op(f"{_NS}::dispatch", mutates_args=())
def dispatch(x: torch.Tensor, topk_w: torch.Tensor, routing_map: torch.Tensor,
             tokens_per_expert: torch.Tensor, padded_offsets: torch.Tensor,
             row_of_slot: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
             num_experts: int, local_begin: int, pad_multiple: int, capacity: int, R: int
             ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    desc, h = _rebuild(routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
                       workspace, num_experts, local_begin, pad_multiple, capacity)
    H = x.shape[1]
    rows = x.new_empty((R, H))
    row_w = x.new_empty(R, dtype=torch.float32)
    row_token = x.new_empty(R, dtype=torch.int32)
    row_expert = x.new_empty(R, dtype=torch.int32)
    B.moe_dispatch(desc, h, x.contiguous(), H, R, rows, topk_w.contiguous(), row_w, row_token,
                   row_expert)
    return rows, row_w, row_token, row_expert


@dispatch.register_fake
def _(x, topk_w, routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
      workspace, num_experts, local_begin, pad_multiple, capacity, R):
    return (x.new_empty((R, x.shape[1])), x.new_empty(R, dtype=torch.float32),
            x.new_empty(R, dtype=torch.int32), x.new_empty(R, dtype=torch.int32))


@torch.library.custom_op(f"{_NS}::dispatch_fp8", mutates_args=())
def dispatch_fp8(x: torch.Tensor, topk_w: torch.Tensor, routing_map: torch.Tensor,
                 tokens_per_expert: torch.Tensor, padded_offsets: torch.Tensor,
                 row_of_slot: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
                 num_experts: int, local_begin: int, pad_multiple: int, capacity: int, R: int
                 ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """FP8 dispatch: (rows_q [R,H] float8_e4m3fn, row_scale [R,H/128] fp32, row_w,
    row_token, row_expert).  Not differentiable (the codes are a quantization)."""
    desc, h = _rebuild(routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
                       workspace, num_experts, local_begin, pad_multiple, capacity)
    H = x.shape[1]
    rows_q = x.new_empty((R, H), dtype=torch.float8_e4m3fn)
    row_scale = x.new_empty((R, H // 128), dtype=torch.float32)
    row_w = x.new_empty(R, dtype=torch.float32)
    row_token = x.new_empty(R, dtype=torch.int32)
    row_expert = x.new_empty(R, dtype=torch.int32)
    B.moe_dispatch_fp8(desc, h, x.contiguous(), H, R, rows_q, row_scale, topk_w.contiguous(),
                       row_w, row_token, row_expert)
    return rows_q, row_scale, row_w, row_token, row_expert


@dispatch_fp8.register_fake
def _(x, topk_w, routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
      workspace, num_experts, local_begin, pad_multiple, capacity, R):
    H = x.shape[1]
    return (x.new_empty((R, H), dtype=torch.float8_e4m3fn),
            x.new_empty((R, H // 128), dtype=torch.float32), x.new_empty(R, dtype=torch.float32),
            x.new_empty(R, dtype=torch.int32), x.new_empty(R, dtype=torch.int32))


@torch.library.custom_op(f"{_NS}::dispatch_bwd", mutates_args=())
def dispatch_bwd(grad_rows: torch.Tensor, grad_row_w: torch.Tensor, routing_map: torch.Tensor,
                 tokens_per_expert: torch.Tensor, padded_offsets: torch.Tensor,
                 row_of_slot: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
                 num_experts: int, local_begin: int, pad_multiple: int, capacity: int
                 ) -> tuple[torch.Tensor, torch.Tensor]:
    desc, h = _rebuild(routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
                       workspace, num_experts, local_begin, pad_multiple, capacity)
    R, H = grad_rows.shape
    T, k = row_of_slot.shape
    grad_x = grad_rows.new_empty((T, H))
    grad_topk_w = grad_rows.new_empty((T, k), dtype=torch.float32)
    B.moe_dispatch_bwd(desc, h, grad_rows.contiguous(), H, R, grad_x, grad_row_w.contiguous(),
                       grad_topk_w)
    return grad_x, grad_topk_w


@dispatch_bwd.register_fake
def _(grad_rows, grad_row_w, routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
      workspace, num_experts, local_begin, pad_multiple, capacity):
    T, k = row_of_slot.shape
    return (grad_rows.new_empty((T, grad_rows.shape[1])),
            grad_rows.new_empty((T, k), dtype=torch.float32))


def _dispatch_setup(ctx, inputs, output):
    x, _, routing_map, tpe, off, ros, status, ws, E, lb, P, cap, R = inputs
    ctx.save_for_backward(routing_map, tpe, off, ros, status, ws)
    ctx.args = (E, lb, P, cap, R, x.shape[1], x.dtype)


def _dispatch_backward(ctx, grad_rows, grad_row_w, _grad_token, _grad_expert):
    routing_map, tpe, off, ros, status, ws = ctx.saved_tensors
    E, lb, P, cap, R, H, dtype = ctx.args
    if grad_rows is None:
        grad_rows = ros.new_zeros((R, H), dtype=dtype)
    if grad_row_w is None:
        grad_row_w = ros.new_zeros(R, dtype=torch.float32)
    grad_x, grad_topk_w = dispatch_bwd(grad_rows, grad_row_w, routing_map, tpe, off, ros, status,
                                       ws, E, lb, P, cap)
    return (grad_x, grad_topk_w) + (None,) * 11


dispatch.register_autograd(_dispatch_backward, setup_context=_dispatch_setup)


# ---------------------------------------------------------------------------
# combine, with autograd through moe_combine_bwd
# ---------------------------------------------------------------------------
@torch.library.custom_op(f"{_NS}::combine", mutates_args=())
def combine(Y: torch.Tensor, routing_map: torch.Tensor, tokens_per_expert: torch.Tensor,
            padded_offsets: torch.Tensor, row_of_slot: torch.Tensor, status: torch.Tensor,
            workspace: torch.Tensor, num_experts: int, local_begin: int, pad_multiple: int,
            capacity: int) -> torch.Tensor:
    desc, h = _rebuild(routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
                       workspace, num_experts, local_begin, pad_multiple, capacity)
    R, H = Y.shape
    out = Y.new_empty((row_of_slot.shape[0], H))
    B.moe_combine(desc, h, Y.contiguous(), H, R, out)
    return out


@combine.register_fake
def _(Y, routing_map, tokens_per_expert, padded_offsets, row_of_slot, status, workspace,
      num_experts, local_begin, pad_multiple, capacity):
    return Y.new_empty((row_of_slot.shape[0], Y.shape[1]))


@torch.library.custom_op(f"{_NS}::combine_bwd", mutates_args=())
def combine_bwd(grad_out: torch.Tensor, R: int, routing_map: torch.Tensor,
                tokens_per_expert: torch.Tensor, padded_offsets: torch.Tensor,
                row_of_slot: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
                num_experts: int, local_begin: int, pad_multiple: int, capacity: int
                ) -> torch.Tensor:
    desc, h = _rebuild(routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
                       workspace, num_experts, local_begin, pad_multiple, capacity)
    H = grad_out.shape[1]
    grad_rows = grad_out.new_empty((R, H))
    B.moe_combine_bwd(desc, h, grad_out.contiguous(), H, R, grad_rows)
    return grad_rows


@combine_bwd.register_fake
def _(grad_out, R, routing_map, tokens_per_expert, padded_offsets, row_of_slot, status,
      workspace, num_experts, local_begin, pad_multiple, capacity):
    return grad_out.new_empty((R, grad_out.shape[1]))


def _combine_setup(ctx, inputs, output):
    Y, routing_map, tpe, off, ros, status, ws, E, lb, P, cap = inputs
    ctx.save_for_backward(routing_map, tpe, off, ros, status, ws)
    ctx.args = (Y.shape[0], E, lb, P, cap)


def _combine_backward(ctx, grad_out):
    routing_map, tpe, off, ros, status, ws = ctx.saved_tensors
    R, E, lb, P, cap = ctx.args
    grad_rows = combine_bwd(grad_out, R, routing_map, tpe, off, ros, status, ws, E, lb, P, cap)
    return (grad_rows,) + (None,) * 10


combine.register_autograd(_combine_backward, setup_context=_combine_setup)


# ---------------------------------------------------------------------------
# a whole expert-parallel layer on one GPU's share
# ---------------------------------------------------------------------------
def moe_layer(x, topk_idx, topk_w, experts, num_experts, local_begin=0, num_local=None,
              pad_multiple=1, capacity=0):
    """Route, dispatch, run ``experts(rows, row_w, row_expert)`` on the
    expanded rows (the experts apply the routing weights), combine.

    Differentiable in x and topk_w.  capacity > 0 selects the sync-free mode
    (R = capacity, pad and sentinel rows zero, capturable and traceable with
    static shapes); capacity == 0 reads the row count back once."""
    num_local = num_experts if num_local is None else num_local
    *handle, host = route(topk_idx, num_experts, local_begin, num_local, pad_multiple, capacity)
    R = capacity if capacity > 0 else int(host[0])
    rows, row_w, _, row_expert = dispatch(x, topk_w, *handle, num_experts, local_begin,
                                          pad_multiple, capacity, R)
    Y = experts(rows, row_w, row_expert)
    return combine(Y, *handle, num_experts, local_begin, pad_multiple, capacity)
