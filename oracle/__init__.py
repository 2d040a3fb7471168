"""Plain, slow fp64 CPU oracle of the Muse Glimmer / Muse Spark Open attention layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
shares no code with that path.

Every function follows the definition the pages give, in their order and
notation, in float64, with NumPy library primitives (matmul, exp, sqrt, sin,
cos) as single steps and no blocking, fusion or reordering:

* weightless per-head RMS QK-norm with eps 1e-5, the fixed query multiplier
  s applied after the norm, and the usual 1/sqrt(d) softmax scale on top
  (Muse Spark Open deep dive, section 3.2, the five-step forward order and
  the logit equation logit = s*sqrt(d)*cos(theta));
* RoPE on local layers only, rotating the whole head with dimension j paired
  with j + d/2 and inverse frequency theta**(-2j/d); global layers get no
  rotation (same page, section 3.4 and its implementation notes);
* causal sliding window: key j is visible to query i iff i - W < j <= i;
  global layers: j <= i (section 3.4, the mask note);
* grouped-query attention: query head h reads KV head floor(h / G)
  (section 3.1, repeat_kv);
* fp64 softmax with the row maximum subtracted;
* Spark's weightless per-head output RMSNorm before the gate, then the
  elementwise sigmoid gate y = o * sigmoid(g) (section 3.3; the
  normalization-and-gates audit on flozi.net, attention paragraph);
* layer schedule: layer i of L is global iff (L - 1 - i) mod 4 == 0
  (section 2.2, the layer-type equation).

Readings where the pages are silent are listed in the repository's design
notes; the ones that matter here: the gate logits are an input tensor
[B, T, Hq, D] (the projection W_G x is outside the layer's hot path); RoPE
uses the positions given (prefill default 0..T-1); in decode the new token
sits at position L - 1 where L counts it, and cached keys are taken exactly
as stored (bf16, already normalized and rotated).  A prefill chunk continuing
a cached sequence reads its history the same way, and its own tokens sit at
positions start .. start + T - 1; a drafter's non-causal block sees the same
history and every block key within the window in both directions.

A flagged second mode (``reference_rounding``) rounds the normalized query,
its product with s, and the normalized key to bf16 where the pages'
reference implementation casts them (section 3.2 implementation notes).  It
is reported beside the plain fp64 oracle and never replaces it.
"""
from .attention import (  # noqa: F401
    layer_is_global,
    global_layers,
    visible_range,
    bidirectional_range,
    visible_mask,
    rms_normalize,
    to_bf16,
    rope_inv_freq,
    rope_rotate,
    query_prologue,
    key_prologue,
    qk_prologue,
    logits_for_row,
    softmax,
    attend_rows,
    output_epilogue,
    sigmoid,
    prefill,
    decode_one,
    prefill_chunk,
    block_bidirectional,
)
from . import fp8  # noqa: F401  (E4M3 cache codes)
from . import block  # noqa: F401  (the attention half of a decoder block)
