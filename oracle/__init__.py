"""CPU oracle for exact scaled-dot-product attention (float64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, table or
helper with the HIP library; the only thing both sides share is the seeded
input generator in ``synth``.

Pages cited (by title and section):

* [BLOG] "AI infra. 一层全看懂(五)Flash Attention:AI编译优化的集大成者"
  (yeyulingfeng.com): §一 the three steps QK^T -> softmax -> PV; §三 the
  standard three-pass attention with its FLOP and byte counts; §四 safe
  softmax (subtract the row maximum) and the tiling notation B_r, B_c.
* [KB] "FlashAttention：为什么少搬数据，反而算得更快" (xuujii.github.io ai-infra-kb,
  M007): §02 the three actions and the note that scale and causal mask are
  part of the real computation; §04 the online-softmax state (m, l, U), its
  update rule, the initial state and the hand-worked example; §05 backward by
  recomputing P from the forward's row statistics; §08 the q/k/v layout
  [batch, heads, sequence, head_dim].
* [NEWS] "FlashAttention技术原理详解：通过内存优化加速注意力计算"
  (news.pikppo.com): MHA / MQA / GQA support.

Modules
-------
``reference``  the definition, written out: S and P materialised, textbook
               softmax, textbook chain rule for the gradients (the oracle
               proper, used for every parity check).
``online``     the blockwise online-softmax recurrence of [KB] §04, used only
               to pin the oracle to the pages' worked example and to show that
               any block size reaches the same result.
``brute``      scalar pure-Python loops for tiny inputs (a second, independent
               spelling of the definition).

``reference.paged_decode_forward`` is decode over a paged K/V cache: the keys
of each sequence gathered through its page-table row, then the definition.
``fp8``        the forward of E4M3 (8-bit float) inputs with per-tensor
               descale factors: their decoded values, then the definition;
               and the bound on what rounding P to E4M3 may change in O.
``bounds``     magnitude sums of the gradients' terms, which bound what
               rounding probabilities and dS to 16 bits may change in them
               (used by the parity tests' element-wise gradient check).
``dropout``    dropout on the probabilities with a mask drawn from the
               counter-based generator Philox4x64-10 (readings in its
               docstring), forward and backward.

Readings of the pages where they are silent are listed in ``reference``.
Parity status: every function here is pinned by a CPU test in
``tests/test_oracle.py``. The one unpinned value is the output O = 0 of a
query row that sees no key at all, a convention the pages leave open ([KB]
§04 says only that such rows must be handled). Its LSE = -inf is pinned as
the log-sum-exp of an empty set (scipy), and its zero gradient by finite
differences of the forward.
"""

from .reference import (  # noqa: F401
    attention_forward,
    attention_backward,
    head_forward,
    head_backward,
    paged_decode_forward,
    paged_gather,
    visible_mask,
)
from .dropout import (  # noqa: F401
    attention_backward_dropout,
    attention_forward_dropout,
    keep_mask,
    keep_scale,
    philox4x64,
    threshold,
)
from .fp8 import decode as fp8_decode, head_forward_fp8, p_rounding_bound  # noqa: F401
from .bounds import (  # noqa: F401
    attention_backward_magnitudes,
    group_backward_magnitudes,
    head_backward_magnitudes,
)
from .online import online_row, online_forward  # noqa: F401
from .brute import brute_forward  # noqa: F401
