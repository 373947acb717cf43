"""Plain, slow CPU oracle for the QLoRA NF4 hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant generator with the HIP library in ``bit_nf4_quantized_22_amd``,
and imports nothing from it.

Modules
  nf4     -- NF4 codebook, blockwise absmax quantisation, double quantisation
             of the block constants, dequantisation (IEEE fp32 where the method
             decides an integer code, fp64 for the codebook construction).
  linear  -- the "4-bit storage, 16-bit compute" linear layer with a LoRA
             bypass: forward, backward to the input, LoRA gradients (fp64).
  memory  -- storage accounting (bits per parameter, LoRA parameter counts).
  optim   -- the AdamW step on the LoRA matrices (fp64).
  dropout -- LoRA dropout on the adapter branch: the counter-based mask
             (Philox4x64-10) and the dropped forward, backward (fp64).
  codebooks -- the FP4 weight table, the FP8 (E4M3) level-2 code, mean-
             centred double quantisation (signed 8-bit code) and the
             uniform INT4 strawman of the error study.

Every function names the page and section it follows.  Pages are cited by
title (site in brackets):
  [rkmt]  "QLORA技术解析：4-bit量化与LoRA结合，单卡微调百亿大模型" (rkmt.cn)
  [czcl]  "QLoRA技術解析：4-bit量化與高效微調實戰" (czchanglian.com)
  [fg8]   "完全开发指南：QLoRA，避坑必备" (faguo8.com)
  [tgd]   "QLoRA微调" (theguodong.com)
  [kwkr]  "【79.PythonAI】QLoRA原理深入：4-bit量化+LoRA，24G显存也能微调7B模型" (kwkr.cn)

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except the agreement of the NF4 table with the
table printed in the original publication, which none of the pages carries
(parity unpinned for that comparison only).
"""

from . import nf4, linear, memory, optim, dropout, codebooks  # noqa: F401
