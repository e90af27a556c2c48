"""CPU oracle for prefix-tree-packed attention and the Basal decision.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP library and imports
nothing from ``prefix_tree_packed_amd``.

It is a plain, slow, obviously correct restatement of what the pages define:

* ``oracle.tree``      index tables and the dense visibility mask of a packed tree
                       (architecture page, section 03 "Packing", "Attention over
                       tree blocks"; section 01 "Batch and prefix tree");
* ``oracle.attention`` dense-mask softmax attention in float64;
* ``oracle.decision``  the two-order decision and temperature calibration
                       (architecture page, section 02 "Basal protocol");
* ``oracle.rope``      rotary position embedding at the tokens' prompt
                       positions (architecture page, section 03; AstrAI's
                       inference guide, "Rotary Embedding Backend", "KV Cache");
* ``oracle.packing``   tokenized prompts into prefix-tree rows, request cost,
                       batch formation (architecture page, sections 01, 03, 04);
* ``oracle.readout``   the last layer's MLP block and answer-letter logits
                       at readout rows only, float16 storage points (architecture
                       page, sections 01 and 05).

"The architecture page" throughout is "How basal-rs computes a decision"
(basal.itsol.dev/en/architecture), with its Polish version
(basal.itsol.dev/pl/architektura) used to read garbled passages; "AstrAI's
inference guide" is the "Inference" guide of the AstrAI repository
(docs/guides/inference.md).

Every function is pinned by ``-m "not gpu"`` tests against the pages' worked
examples, closed forms, invariants and brute force; none is "parity unpinned".
"""
from . import tree, attention, decision, rope, packing, readout  # noqa: F401
