"""Plain, slow, f64 CPU oracle for split-KV matrix-absorbed MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs
anything in this package: only the tests, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. It shares no code with the HIP library (``absorbed_mla_paged_amd``); both
sides take their inputs from the seeded generator in ``mla_synth``.

What it computes, and where each piece comes from:

* ``reference.latent_f64`` -- the single-pass answer: per request and head,
  softmax over every cached token of scale*(q_absorbed.ckv + q_pe.kpe),
  weights applied to the 512-wide ckv rows, plus the base-2 log-sum-exp.
  (mlxcel pull request 995, "What changed", the Stage 1 bullet: the rope
  half of the score is an additive term next to the latent half, one scale
  over both, and values are the latent rows themselves.)
* ``reference.decompressed_f64`` -- the pre-absorption computation: per head,
  keys W_UK.ckv (+ kpe), values W_UV^T applied to ckv, ordinary softmax
  attention. (mlxcel pull request 995, "What changed", the absorb.rs bullet
  for the W_UK / W_UV^T shapes; "Verified vs unverified" for a host f64
  reference that performs the pre-absorption computation.)
* ``reference.partials_f64`` / ``merge_log2_f64`` -- split-KV: each chunk of
  the context yields a normalised partial and its log2 LSE, and the merge
  weights partials by 2^(lse2 - max). (vllm-metal pull request 601 "[kernel]
  Wire MLA split-KV decode", "What changed"; mlxcel pull request 995, "How
  #898's merge kernel is reused", for the log2 clause.)
* ``reference.merge_ln_wrong`` -- the negative control: natural-log LSEs fed
  to the log2 merge (same section of mlxcel pull request 995).
* ``plan.*`` -- an independent mirror of the host partition chooser and the
  partition/tile index math (vllm-metal pull request 601, "What changed",
  the dispatch gates).
* ``brute.*`` -- 50-digit mpmath scalar loops over the literal definitions,
  used to pin the f64 functions on tiny inputs.
* ``byte_model`` -- KV bytes per token, latent vs decompressed (mlxcel pull
  request 995, commit "performance-validation report").
* ``reference.decode_fp8_e4m3`` -- E4M3 bytes to values, from the E4M3
  definition of the OCP 8-bit floating point specification, for latent
  caches stored in 8 bits with one scale (the pages keep 16-bit caches and
  decline others; this cache variant and its single scale are our reading).

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, brute force, invariances, the pages'
printed byte counts). None is "parity unpinned".
"""
from .reference import (LOG2_E, decode16, decode_fp8_e4m3, gather_request, latent_f64,
                        latent_one, decompressed_f64, absorb_query,
                        unabsorb_output, partials_f64, merge_log2_f64,
                        merge_ln_wrong, orthogonal_weights)
from .plan import (PlanParams, choose_partitions, partition_range,
                   row_ranges, default_heads_per_wg)
from .byte_model import (latent_bytes_per_token, decompressed_bytes_per_token,
                         max_context_tokens)

__all__ = [
    "LOG2_E", "decode16", "decode_fp8_e4m3", "gather_request", "latent_f64", "latent_one",
    "decompressed_f64", "absorb_query", "unabsorb_output", "partials_f64",
    "merge_log2_f64", "merge_ln_wrong", "orthogonal_weights", "PlanParams",
    "choose_partitions", "partition_range", "row_ranges",
    "default_heads_per_wg", "latent_bytes_per_token",
    "decompressed_bytes_per_token", "max_context_tokens",
]
