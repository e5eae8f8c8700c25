"""Plain fp64 CPU oracle for one D2F denoising step.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``, and by
nothing else.  The HIP library never calls it, and it shares no code with the
library: it is written from the pages' description of the method, in numpy
float64, with no tiling, fusion or reordering beyond what the definitions
state.

Sources (cited by page title and section; the short names are used below):

* [D2F-wiki]    "D2F: 확산 언어 모델이 KV 캐시를 얻고 자기회귀 모델보다 2.5배
                빨라지는 방법 (arXiv:2508.09192)", llm-wiki.hwlabs.dev.
* [D2F-review]  "D2F 논문 리뷰: 확산 LLM이 자기회귀 모델보다 빠른 추론을 처음으로
                달성한 방식", allinfo.ai.kr.
* [dLLM-survey] "확산 언어 모델(Diffusion LLM)이란 무엇인가", discuss.pytorch.kr.

Modules:
  attention  block-causal window attention over a frozen cache (contiguous or paged)
  commit     per-position confidence/argmax and the block commit rule
  kv_cache   appending a completed block to the cache
  window     the active-window schedule of pipelined decoding

Every function here is pinned by a CPU test against something other than
itself (closed forms, library routines on special cases, invariants, brute
force, hand-worked fixtures); see ``tests/test_oracle_*.py``.
"""
from . import attention, commit, kv_cache, window  # noqa: F401
from .common import as_f64  # noqa: F401
