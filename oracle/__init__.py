"""CPU oracle for the fused attention forward and the latent-cache MLA decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library never imports, links or calls anything here, and
nothing here imports the HIP library: the two share no code.  Inputs arrive as
numpy arrays (already rounded to the precision the GPU received) and every
computation runs in float64 with plain numpy primitives.

Modules
-------
``attention``  explicit softmax attention (the definition), the tiled online
               softmax written out in the blog's order of steps, and the
               blog's causal tile-range arithmetic.
``mla``        absorbed latent-cache decode, weight absorption, explicit
               key decompression (the unfused comparison path), split partials
               and the log-sum-exp combine.
``plan``       the split-KV work plan of the decode scheduler, in plain loops.

Citation key used in the docstrings (pages, not files):
  [FA2-v2 blog]    blog post implementing a FlashAttention-2 style "v2"
                   fp32 forward on CUDA cores (RTX 5080); sections 1.1-5.
  [MLA-FA3 article] article on fusing MLA with FlashAttention-3 on Hopper;
                   sections: fused dataflow figure, section 1 (TMA descriptor),
                   section 2 (warp-specialised WGMMA in-place absorption,
                   absorption equation), benchmark table.
  [FlashMLA #26]   GitHub issue listing ten optimisation ideas for FlashMLA.

Parity status of every public function is stated in its docstring
("pinned by: ..."); no function here is parity unpinned.
"""

from .attention import (  # noqa: F401
    attn_ref,
    online_attn_ref,
    causal_kv_tiles,
    is_diagonal_tile,
    v2_shared_bytes,
    v2_launch_shape,
)
from .mla import (  # noqa: F401
    mla_decode_ref,
    absorb_ref,
    decompress_k_ref,
    mla_decode_explicit_ref,
    split_partials_ref,
    combine_ref,
    round_bf16,
    absorb_decode_ref,
)
from .plan import plan_ref, plan_pieces_ref, plan_slot_ref  # noqa: F401
