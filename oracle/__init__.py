"""CPU oracle for exact scaled-dot-product attention (FlashAttention).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library under ``exact_attention_25_amd/`` and imports nothing from it.

Everything here is plain numpy in float64 (pure Python for the brute force),
written from the definitions on these pages (cited by title and section):

* [FA-CUDA]  "CUDA FlashAttention: from online softmax to the long-sequence IO
  limit" (chengzipai.xyz) -- §1 problem definition and causal mask, §4 the
  online-softmax merge, §6 state-ordering rules.
* [FA-ALGO]  "FlashAttention algorithm details: forward/backward tiling, online
  softmax, cumulative update and numerical stability" (5688vip.com, ch. 4) --
  §4.2.1-4.2.2 forward tiling and recurrence, §4.3.1 backward formulas.
* [FA-WHY]   "Why FlashAttention does not need to store the attention matrix"
  (jefxiong.cn) -- §3.1 safe softmax, §3.2 online recurrence and LSE, §3.3
  backward with the scale factor, §4.5 causal block skipping, §05 dropout
  regenerated from the Philox seed and offset.
* [FA-MI50]  "FlashAttention dataflow and engineering validation on MI50"
  (mpbf.cn/news/61284) -- §2.2 worked example, §3.3 backward correction term,
  §4.3 block-level flags of padding masks, §5.1 random mask patterns.

Modules
-------
``attention``  plain-definition forward / backward (materialised rows,
               optional key-padding mask, grouped K/V heads, dropout),
               online tiled forward, state merge, key-split partial states,
               block-level mask flags, pure-Python brute force.
``dropout``    Philox4x64-10 and the dropout keep mask regenerated from
               (seed, offset).

Every function in ``attention`` is pinned by ``tests/test_oracle.py``; none is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_probs,
    online_forward,
    merge_states,
    attention_partial,
    merge_lse,
    brute_force_forward,
    causal_tile_count,
    key_tile_words,
)
from .dropout import (  # noqa: F401
    dropout_keep,
    dropout_keep_rows,
    dropout_threshold,
    philox4x64,
    philox4x64_array,
)
