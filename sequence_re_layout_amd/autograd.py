"""torch.autograd wrappers of the attention-boundary re-layouts.

A training step needs the re-layouts on both passes.  The gradient of a
permutation is its inverse, so each forward call's backward is the library's
call in the other direction (include/basp.h, "Backward pass of the same
boundary"):

* ``seq_to_head_qkv(plan, q, k, v)`` runs ``basp_seq_to_head`` (fused Q, K, V
  sequence-sharded -> head-sharded) and, on the backward pass,
  ``basp_head_to_seq_qkv`` (the fused gradient head-sharded -> dQ, dK, dV
  sequence-sharded);
* ``head_to_seq_o(plan, o)`` runs ``basp_head_to_seq`` (attention output
  head-sharded -> sequence-sharded) and, on the backward pass,
  ``basp_seq_to_head_o`` (dO sequence-sharded -> head-sharded).

Tensors are flat, contiguous and of the plan's dtype and element counts, as
the binding checks; outputs are allocated with torch on the inputs' device.
Only buffers are marshalled here: every element is moved by the library's
kernels.
"""
from __future__ import annotations

import torch

from . import binding as b


class _SeqToHeadQKV(torch.autograd.Function):
    @staticmethod
    def forward(ctx, plan, q, k, v):
        i = plan.info
        out = torch.empty(i["qkv_elems"], dtype=q.dtype, device=q.device)
        b.basp_seq_to_head(plan, q, k, v, out)
        ctx.plan = plan
        return out

    @staticmethod
    def backward(ctx, grad):
        i = ctx.plan.info
        dev, dt = grad.device, grad.dtype
        dq = torch.empty(i["q_elems"], dtype=dt, device=dev)
        dk = torch.empty(i["kv_elems"], dtype=dt, device=dev)
        dv = torch.empty(i["kv_elems"], dtype=dt, device=dev)
        b.basp_head_to_seq_qkv(ctx.plan, grad.contiguous(), dq, dk, dv)
        return None, dq, dk, dv


class _HeadToSeqO(torch.autograd.Function):
    @staticmethod
    def forward(ctx, plan, o):
        out = torch.empty(plan.info["q_elems"], dtype=o.dtype, device=o.device)
        b.basp_head_to_seq(plan, o, out)
        ctx.plan = plan
        return out

    @staticmethod
    def backward(ctx, grad):
        do = torch.empty(ctx.plan.info["q_elems"], dtype=grad.dtype, device=grad.device)
        b.basp_seq_to_head_o(ctx.plan, grad.contiguous(), do)
        return None, do


def seq_to_head_qkv(plan, q, k, v):
    """Fused Q/K/V seq -> head with its backward (see the module docstring).
    Returns the head-sharded HEAD(Q) || HEAD(K) || HEAD(V) buffer."""
    return _SeqToHeadQKV.apply(plan, q, k, v)


def head_to_seq_o(plan, o):
    """Attention output head -> seq with its backward (see the module
    docstring).  Returns the sequence-sharded output."""
    return _HeadToSeqO.apply(plan, o)
