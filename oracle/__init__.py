"""CPU oracle for the speculative-sampling verify step (test infrastructure only).

This package is a plain, slow, fp64 NumPy statement of what the verify step
computes.  It exists to check the HIP library against the pages that define the
method.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does.  The oracle's arithmetic shares no
code with the product package: the only import from it is the seeded input generator
(rejection_sampling_verify_chain_amd.inputs, which holds none of the method's
arithmetic), and only the calibration script calibrate_zipf_sigma.py uses it, to draw
the workload it calibrates.

Sources (cited by page title and section throughout):

* "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
  (0h-n0.github.io explainer of arXiv:2302.01318) — chain verification:
  Step 2 (ステップ2), Step 3 (ステップ3) accept equation, modified rejection
  sampling (修正付き棄却サンプリング) equation, expected speedup
  (期待される高速化) equation, the sequence diagram and the code sketch.
* "投機的デコーディングとは？LLMの回答を高速化する仕組み"
  (ai-compass.weeybrid.co.jp) — greedy verification and the worked example
  (候補の採用と棄却を具体例で見る).
* SpecInfer article (abeam.tech, arXiv:2305.09781) — token-tree verification:
  basic idea (基本アイデア) and inference (推論方法).
* The ai-compass page's worked example also defines greedy chain verification
  (oracle/greedy.py): accept drafts while they equal the target's argmax.
* Per-position acceptance rates (oracle/alpha.py): the Speculative Sampling explainer's
  Step 3 accept probability averaged over the drafted token.
* The draft-side sampler (oracle/sample.py): Step 1 and the code sketch's draft loop.
* Accepted-path KV compaction (oracle/kv.py): the explainer's KV-cache rollback note and
  SpecInfer's append of the verified run.

Pins: every function here is checked by the CPU tests against facts that do not
come from this package (Theorem 1 by chi-square, the closed form for the
expected tokens per round, brute-force tree enumeration, library routines for
the special cases, and the worked examples under tests/golden/).
"""

from .chain import (  # noqa: F401
    ROW_TOKEN_RANGE, ROW_NONFINITE, ROW_RESIDUAL_ZERO, ROW_BAD_TREE,
    ROW_BAD_TEMPERATURE, ROW_BAD_UNIFORM, FALLBACK_BITS, BAND,
    widen, softmax_fp64, inverse_cdf, draw_band, verify_chain_seq, verify_chain_batch,
)
from .tree import argmax_first, verify_tree_one, verify_tree_batch  # noqa: F401
from .greedy import verify_chain_greedy_seq, verify_chain_greedy_batch  # noqa: F401
from .alpha import acceptance_rate, acceptance_rates_seq, acceptance_rates_batch  # noqa: F401
from .sample import sample_row, sample_batch  # noqa: F401
from .kv import ROW_BAD_INDEX, compact_one, compact_batch  # noqa: F401
