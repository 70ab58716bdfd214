"""Autograd functions over the C ABI, for training.

- The Ulysses relayout moves values without arithmetic, so its gradient is the
  inverse relayout: seq->head's backward is head->seq of the upstream gradient
  and the other way round, bit for bit (FastVideo "[perf] Probe H3 chunked
  all-to-all with direct output slices", benchmark_ulysses_a2a.py: the
  forward/backward training pair, whose gradients must equal the collective's
  exactly).  The same holds for the cu_seqlens varlen relayout and for the
  relayout over a THD layout plan's spans.
- The stable combine's gradient is lse_combine_backward (cuLA PR "feat
  (distributed): add packed hybrid runtime and THD planner", Validation: the
  forward and backward of context parallelism compared against a reference).

Each function only marshals arguments; forward and backward both run in the
HIP kernels behind the C ABI.
"""

from __future__ import annotations

import torch

from . import (ThdPlan, VarlenPlan, lse_combine_backward, ulysses_head_to_seq, ulysses_head_to_seq_spans,
               ulysses_head_to_seq_varlen, ulysses_seq_to_head, ulysses_seq_to_head_spans, ulysses_seq_to_head_varlen)
from . import lse_combine as _lse_combine
from . import lse_combine_planned as _lse_combine_planned
from . import lse_combine_varlen as _lse_combine_varlen

__all__ = ["seq_to_head", "head_to_seq", "seq_to_head_varlen", "head_to_seq_varlen", "seq_to_head_spans",
           "head_to_seq_spans", "lse_combine"]


class _SeqToHead(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, P):
        ctx.P = P
        return ulysses_seq_to_head(x.contiguous(), P)

    @staticmethod
    def backward(ctx, g):
        return ulysses_head_to_seq(g.contiguous(), ctx.P), None


class _HeadToSeq(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, P):
        ctx.P = P
        return ulysses_head_to_seq(x.contiguous(), P)

    @staticmethod
    def backward(ctx, g):
        return ulysses_seq_to_head(g.contiguous(), ctx.P), None


class _SeqToHeadVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, plan, B):
        ctx.plan = plan
        return ulysses_seq_to_head_varlen(x.contiguous(), plan, B)

    @staticmethod
    def backward(ctx, g):
        return ulysses_head_to_seq_varlen(g.contiguous(), ctx.plan), None, None


class _HeadToSeqVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, plan):
        ctx.plan = plan
        ctx.B = x.shape[1]
        return ulysses_head_to_seq_varlen(x.contiguous(), plan)

    @staticmethod
    def backward(ctx, g):
        return ulysses_seq_to_head_varlen(g.contiguous(), ctx.plan, ctx.B), None


class _SeqToHeadSpans(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, plan, B):
        ctx.plan = plan
        return ulysses_seq_to_head_spans(x.contiguous(), plan, B)

    @staticmethod
    def backward(ctx, g):
        return ulysses_head_to_seq_spans(g.contiguous(), ctx.plan), None, None


class _HeadToSeqSpans(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, plan):
        ctx.plan = plan
        ctx.B = x.shape[1]
        return ulysses_head_to_seq_spans(x.contiguous(), plan)

    @staticmethod
    def backward(ctx, g):
        return ulysses_seq_to_head_spans(g.contiguous(), ctx.plan, ctx.B), None


class _LseCombine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, part_out, part_lse, cu_seqlens, plan):
        if plan is not None:
            out, lse = _lse_combine_planned(part_out, part_lse, plan)
        elif cu_seqlens is None:
            out, lse = _lse_combine(part_out, part_lse)
        else:
            out, lse = _lse_combine_varlen(part_out, part_lse, cu_seqlens)
        ctx.save_for_backward(part_out, part_lse, cu_seqlens)
        ctx.plan = plan
        return out, lse

    @staticmethod
    def backward(ctx, g_out, g_lse):
        part_out, part_lse, cu_seqlens = ctx.saved_tensors
        if g_out is None:
            g_out = torch.zeros(part_out.shape[1:], dtype=part_out.dtype, device=part_out.device)
        elif g_out.stride(-1) != 1 or g_out.dtype != part_out.dtype:
            g_out = g_out.to(part_out.dtype).contiguous()
        if g_lse is not None and g_lse.dtype != torch.float32:
            g_lse = g_lse.float()
        d_po, d_pl = lse_combine_backward(part_out, part_lse, g_out, g_lse, cu_seqlens, plan=ctx.plan)
        return d_po, d_pl, None, None


def seq_to_head(x: torch.Tensor, P: int) -> torch.Tensor:
    """Differentiable ulysses_seq_to_head: [P][B][S/P][H][D] -> [P][B][S][H/P][D]."""
    return _SeqToHead.apply(x, P)


def head_to_seq(x: torch.Tensor, P: int) -> torch.Tensor:
    """Differentiable ulysses_head_to_seq: [P][B][S][H/P][D] -> [P][B][S/P][H][D]."""
    return _HeadToSeq.apply(x, P)


def seq_to_head_varlen(x: torch.Tensor, plan: VarlenPlan, B: int = 1) -> torch.Tensor:
    """Differentiable ulysses_seq_to_head_varlen: rank-major [B*T][H][D] -> [P][B][T][H/P][D]."""
    return _SeqToHeadVarlen.apply(x, plan, B)


def head_to_seq_varlen(x: torch.Tensor, plan: VarlenPlan) -> torch.Tensor:
    """Differentiable ulysses_head_to_seq_varlen: [P][B][T][H/P][D] -> rank-major [B*T][H][D]."""
    return _HeadToSeqVarlen.apply(x, plan)


def seq_to_head_spans(x: torch.Tensor, plan: ThdPlan, B: int = 1) -> torch.Tensor:
    """Differentiable ulysses_seq_to_head_spans: planned slabs [B*T][H][D] -> [P][B][T][H/P][D]."""
    return _SeqToHeadSpans.apply(x, plan, B)


def head_to_seq_spans(x: torch.Tensor, plan: ThdPlan) -> torch.Tensor:
    """Differentiable ulysses_head_to_seq_spans: [P][B][T][H/P][D] -> planned slabs [B*T][H][D]."""
    return _HeadToSeqSpans.apply(x, plan)


def lse_combine(part_out: torch.Tensor, part_lse: torch.Tensor, cu_seqlens: torch.Tensor | None = None,
                plan: ThdPlan | None = None):
    """Differentiable stable combine (causal varlen when cu_seqlens is given,
    causal over a THD layout plan when plan is given): part_out [P][T][H][D],
    part_lse [P][T][H] -> (out [T][H][D], lse_out [T][H])."""
    return _LseCombine.apply(part_out, part_lse, cu_seqlens, plan)
