"""CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package; the library's own path never does and shares no code with it.

Everything here is plain, slow and written to be checked by eye against the
pages: numpy in float64, one library primitive per step (matmul, exp,
cumsum), no blocking or fusion.  Sources (cited by page and section):

* self-speculative decoding page (m.lqnn.cn/news/278124): layer-skip draft
  §2.1, final norm before the head §3.1, KV reuse and rollback §3.3, draft /
  verify / accept-or-reject §4.2-§4.3, lossless rule §2.4, expected-yield
  formula §3.2, losslessness check §5.2.
* "DSpark" page (0539edu.com/news/4524681): greedy block verification §2.1,
  confidence score §2.2, K schedule §2.3, speedup estimate §2.4.
* "FlashSpec" page (lnrk.cn/news/47842): tree batch in level order with a
  parent mask §2.2, per-node position ids §3.2, masked padding §5.2.
* "推测解码技术原理与实践" page (intelliparadigm.com): min(1, p/q) acceptance,
  left-to-right, first reject ends the round §2.2.
"""
