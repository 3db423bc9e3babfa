"""The whole FOCUS step composed from the oracle's functions (test use only).

Order as in the FOCUS paper (Section 4.2 and Figure 5): importance delta of
layers 0/1 -> top-K masked tokens -> gather of the kept hidden rows; then,
for a later layer, the kept rows' new K/V are written into the exact cache
and the kept queries attend over prefix + block (App. E.2.4).

Inputs are host numpy arrays. bf16 tensors arrive as their raw 16-bit
patterns (uint16) so that gather and scatter stay byte copies; attention
widens those patterns to float64 exactly.
"""
from __future__ import annotations

import numpy as np

from .attention import reduced_attention
from .focus import focus_importance_delta
from .rows import gather_rows, kv_scatter
from .selection import topk_select


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def focus_step(*, q0, k0, q1, k1, decoded, k, hidden_rows, pool_kernel, new_k, new_v, q_kept,
               cache_k, cache_v, seq_start, kv_len, row_base, hq, hkv, k_max, scale):
    """Returns dict(delta, idx, count, cu, gathered, cache_k, cache_v, out)."""
    delta = focus_importance_delta(q0, k0, q1, k1, decoded, hq, hkv, pool_kernel)
    idx, count, cu = topk_select(delta, k, k_max)
    gathered = gather_rows(hidden_rows, idx, count, cu)
    ck, cv = kv_scatter(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v)
    as_f = (lambda a: bf16_bits_to_f64(a)) if ck.dtype == np.uint16 else (lambda a: a)
    out = reduced_attention(as_f(q_kept[: int(cu[-1])]), count, cu, as_f(ck), as_f(cv), seq_start,
                            kv_len, hq, hkv, scale)
    return dict(delta=delta, idx=idx, count=count, cu=cu, gathered=gathered, cache_k=ck,
                cache_v=cv, out=out)
