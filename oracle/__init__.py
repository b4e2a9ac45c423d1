"""CPU oracle for compressed sparse attention (c4a / c128a CSA) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The GPU library never calls
it, and it shares no code, header, table or constant generator with the GPU
path: its only common ground with the GPU path is the seeded inputs of
``synth``.

Everything here is plain numpy in float64, written from the definitions on the
three source pages:

* [P1] "vLLM DeepSeek V4 Support: Efficient Long-context Attention"
  (agentlenshq.com), sections "DeepSeek V4 Attention Architecture",
  "KV Cache Memory Management", "GPU Compute Saturation".
* [P2] "vLLM解密：DeepSeek-V4本地部署為何如此困難" (yhxrc.cn), sections
  "二、注意力機制為什么這么麻煩" (attention design), "3.1 顯存" (memory) and
  "3.2 內核" (kernels).
* [P3] blog.hotdry.top, "DeepSeek V4 inference latency optimization"
  (2026-04-24), sections "KV 缓存压缩" (KV compression), "注意力计算剪枝"
  (attention pruning), "工程实现" (engineering).

Where the pages are silent the oracle takes the readings listed in the module
docstrings (labelled R1..R24); the GPU path takes the same ones.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines (torch CPU casts, torch SDPA), brute
force in pure Python and invariants. Fidelity to the real DeepSeek-V4 model
(logit semantics, RMSNorm epsilon, RoPE pairing, joint softmax, softmax scale)
is a convention the pages do not fix: parity unpinned against the real model.
"""
from . import codecs, paging, rope, compress, index, attend, memory_model, output_quant, prepare  # noqa: F401
