"""CPU oracle for one tensor-parallel rank's share of a Llama-style MLP.

TEST INFRASTRUCTURE ONLY.  This package is the independent, slow and
obviously-correct reference that the HIP library is checked against.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``tensor_transformer_mlp_tp_amd``)
never imports, calls or links anything here, and nothing here imports the
product path: the two share no code.  The only module both sides use is
``workloads`` (seeded synthetic inputs), which holds none of the MLP's
arithmetic.

Everything is computed in float64 with numpy from the exact bytes the GPU
receives (bf16 bit patterns, fp32 values, OCP e4m3fn codes plus fp32 scales).

Sources (the web pages the oracle follows):

* "Build a model sharding system for serving 70B+ parameter models"
  (scalablesystem.dev), section "The Tensor-Parallel Shard Group": the
  column-parallel gate/up projections, the row-parallel down projection whose
  per-rank output is a partial sum, and the all-reduce that adds the partials.
* "Tensor, Pipeline and Expert Parallelism: One Model, Many GPUs" (vidyal.ai),
  section "Step 1: tensor parallelism slices every layer": the first matrix is
  split by columns and the activation applied locally; Llama adds a second
  input matrix split the same way; the second matrix is split by rows.
* "Chapter 12 Parallelism Strategies" (arunshar.com), section 12.2.1
  "Tensor Parallelism (Megatron-Style)": A = [A_1 | ... | A_t],
  B = [B_1; ...; B_t], Z = sum_k Z_k.
* "Model, Tensor & Pipeline Parallelism" (engineer-atlas.dev), sections
  "What must remain true about the layout" and "What must stay true after
  deployment": the split must compute the same function as the unsplit
  model, checked split-against-unsplit on a small configuration.
* The same chapter, section 12.3.1 "Sequence Parallelism for LayerNorm and
  Dropout": under sequence parallelism the all-reduce becomes a
  reduce-scatter (rank k keeps the reduced rows of its sequence slice) and
  the next column-parallel projection reads the all-gathered sequence.
* ``oracle/w8a8.py``: the fp8 x fp8 forward (per-token activation codes;
  steps and their order in that file's docstring).
* ``oracle/attn.py``: the attention block's projections under the same split
  (TPAttentionBlock of the scalablesystem.dev section above; heads per rank
  in section 12.2.1 of the arunshar.com chapter; grouped-query KV heads split
  or replicated per "The KV cache splits too, until it doesn't" on the
  vidyal.ai page).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, a library special case, the Megatron invariant,
format tables).  No function is "parity unpinned".
"""

from .formats import (bf16_bits_to_f64, e4m3fn_to_f64, int8_to_f64, e4m3fn_encode, bf16_round_bits,
                      E4M3FN_MAX)
from .w8a8 import quantise_rows_e4m3, dequantise_rows, rank_partial_w8a8_from_storage
from .attn import (
    local_heads,
    head_rows,
    qkv_rank_weight,
    o_proj_rank_weight,
    linear,
    linear_from_storage,
)
from .mlp import (
    silu,
    mlp_full,
    mlp_partial,
    shard_slice,
    shard_of_full,
    fold_fp32,
    gather_rows,
    reduce_scatter_fp32,
    rank_partial_from_storage,
    rms_normalised_max_error,
)

__all__ = [
    "local_heads",
    "head_rows",
    "qkv_rank_weight",
    "o_proj_rank_weight",
    "linear",
    "linear_from_storage",
    "bf16_bits_to_f64",
    "e4m3fn_to_f64",
    "int8_to_f64",
    "e4m3fn_encode",
    "bf16_round_bits",
    "quantise_rows_e4m3",
    "dequantise_rows",
    "rank_partial_w8a8_from_storage",
    "E4M3FN_MAX",
    "silu",
    "mlp_full",
    "mlp_partial",
    "shard_slice",
    "shard_of_full",
    "fold_fp32",
    "gather_rows",
    "reduce_scatter_fp32",
    "rank_partial_from_storage",
    "rms_normalised_max_error",
]
