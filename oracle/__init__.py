"""CPU oracle for the block stage and the flow-matching loop.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never imports it, links it or calls it, and it shares no code with the GPU
library (no kernels, headers, tables or helpers).  The seeded input generator
(``synth``) is the only thing both sides use.

What it computes is the plain, unfused definition, written from the pages:

  [RT] reading note on "Running VLAs at Real-time Speed" (Ma et al.,
       arXiv:2510.26742v1): model structure (§2, Fig. 4), RMSNorm gain
       (§4.1), action/time embedding (§4.2), fused QKV and RoPE (§4.3),
       gated FFN, residual and RMS statistics (§5), roofline (§6.2).
  [PS] AREX Feed article on PhysisServe: a stage is one Transformer block at
       one denoise step; a chunk reads the cached (noisy) KV of earlier
       chunks (section on splitting the pipeline per block and step).

Every function takes a ``dtype`` (float32 by default, float64 for the twin).
Inputs are cast to that dtype and every operation runs in it; bf16 inputs
arrive already widened exactly to float32.

Pins (tests/test_oracle_pins.py) tie each function to something outside
itself: fold identities, brute force, closed forms, torch CPU library
routines, RoPE invariants and the pages' parameter counts.  The whole-block
and whole-loop compositions are pinned through their parts plus float64 torch
re-compositions built from library primitives (rms_norm,
scaled_dot_product_attention, linear, silu): the block on its own, and the
loop over two layers and three Euler steps with distinct per-layer weights and
cached prefixes.  Several streams on one block's weights are independent
applications of block_forward, one per stream with its own cache.  Beyond
these compositions the values are parity unpinned, because the pages print no
worked numeric example.
"""
from .block import (rms_norm, rope_tables, apply_rope, attention, gated_ffn,
                    block_forward)
from .flow import (silu, time_embedding, suffix_embed, velocity_head, euler_integrate,
                   flow_denoise)

__all__ = [
    "rms_norm", "rope_tables", "apply_rope", "attention", "gated_ffn", "block_forward",
    "silu", "time_embedding", "suffix_embed", "velocity_head", "euler_integrate",
    "flow_denoise",
]
