"""CPU oracle for the hybrid compressed attention hot path (CSA + HCA + SWA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The GPU
product path never calls it and shares no code with it.

It is a plain, slow, obviously-correct numpy implementation in float64 of what
the DeepSeek-V4 pages say the attention stack computes:

* "Why DeepSeek V4 Stands Apart" (besthub.dev), Core Architectural
  Innovations: a 128-token sliding window; CSA compresses KV entries 4x and
  keeps the top-1024 (Pro) / top-512 (Flash) entries per query; HCA
  compresses 128:1 and attends densely over all compressed entries.
* "DeepSeek-V4" (atlas.lewiswon.me), Design overview and Core block: CSA
  compresses every 4 tokens into two overlapping streams and scores entries
  with the V3.2 lightning indexer; HCA uses m'=128; RMSNorm on queries and
  compressed KV entries; attention sinks; Inference efficiency: one shared KV
  head (MQA).

Where the pages leave a step open, the oracle takes the plainest reading the
rest supports and states it in the module that uses it.  Modules:

* ``numerics``  rounding to the storage precisions (bf16 / fp32)
* ``compress``  softmax-weighted window pooling + RMSNorm      (kv_compress)
* ``indexer``   lightning-indexer scores + exact top-k         (csa_index_topk)
* ``attention`` partial softmax attention, sink, LSE merge     (csa_sparse_attn,
                hca_attn, swa_merge)
* ``rope``      partial rotary position embedding (last 64 dims; -i on outputs)
* ``pipeline``  the decode / prefill step composed from the above
* ``dense``     a second, independent formulation (one masked softmax over every
                candidate key) used to pin the first one on tiny inputs
"""
from . import numerics, compress, indexer, rope, attention, pipeline, dense  # noqa: F401
