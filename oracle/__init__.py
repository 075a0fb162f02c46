"""fp64 CPU oracle for MQA / GQA / MLA-absorbed attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library never calls it, and it shares no code with the HIP path.

Every function here is the plain definition written out in float64 numpy,
with the key/value broadcast materialised explicitly, so that each step can
be checked against the pages by eye.  Sources (page title, section):

* single-head attention: "带你了解Attention,从MHA到DeepSeek" (api.makesence.top),
  §1.2 -- score = q.k, divide by sqrt(d_k), softmax, weighted sum of values.
* causal mask and the prefill/decode split: "GQA和MLA详解" (lzwjava.github.io),
  §1 "T 出现在哪里".
* GQA head sharing (repeat_interleave along the head axis): same page §2, and
  "Full 路线：保留 softmax，压缩 K/V 表示" (walkerchi.com) §三 (``repeat_kv``).
* MQA as the one-KV-head case: zdabc.icu article on DeepSeek V4.1's head_dim=512
  MQA operator, section "head_dim = 512 为什么值得注意"; makesence §3.1.
* MLA latent cache, matrix absorption and decoupled RoPE key: lzwjava §3,
  makesence §4.3 and §4.5, walkerchi §四 4.2-4.3.
* the steps around absorbed MLA decode -- query absorption, RoPE of the
  decoupled part (``apply_rotary_pos_emb`` as walkerchi §四 4.2 calls it),
  output up-projection: lzwjava §3, walkerchi §四 4.2-4.3.
* MLA prefill in the expanded (MHA) form and decode in the absorbed form:
  makesence §4.4; sparse (top-k) attention over the MLA cache: makesence §5.1.
* chunked prefill (queries = the last T of S tokens, bottom-right causal
  mask): a reading; the pages show only the square mask (lzwjava §1).

Parity status: every function is pinned by ``tests/test_oracle.py``
(brute force, closed forms, invariants, page values); none is unpinned.
"""

from .attention_ref import (  # noqa: F401
    absorb_query,
    decode_ref,
    kv_values_per_token,
    lse_merge,
    mla_absorbed_ref,
    mla_explicit_ref,
    mla_sparse_ref,
    output_project,
    partial_ref,
    prefill_ref,
    prefill_rows_ref,
    repeat_kv_heads,
    rope_ref,
)
