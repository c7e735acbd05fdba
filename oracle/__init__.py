"""CPU oracle for the MoE-layer forward: plain, slow, obviously-correct numpy.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the test suite, the smoke check of the entry module and the CPU-baseline leg of
the benchmark may import or call it.  It shares no code with the HIP path:
both sides read their inputs from ``moe_inputs`` and nothing else.

Stages (pages cited by title and section):
  route     - affinities sqrt(softplus(logit)), bias-adjusted node-limited
              top-k, renormalised gate weights  (mastering-deepseek-v4
              "MoE + Expert-Parallel Overlap", Implemented; zenaique "MoE
              node-limited routing", definition)
  dispatch  - per-expert histogram, exclusive scan, stable permutation into an
              expert-contiguous buffer (deepmox ch.5 "The network becomes part
              of the forward pass"; zenaique "Why all to all dominates")
  ffn       - SwiGLU experts and the shared expert (mastering-deepseek-v4,
              Implemented: 6*d*d_ff flops per token-expert pair)
  combine   - gate-weighted sum back in token order (deepmox ch.5)
  fp8       - e4m3 block quantisation for the fp8 workload
  hash_route - hash router: experts fixed by a Philox hash of the token id
              (mastering-deepseek-v4, Implemented: hash router for early layers)
  backward  - the layer's backward: combine, expert dgrad/wgrad, dispatch and
              gate gradients (deepmox ch.5: the backward splits into input and
              weight gradients and carries its own exchanges)
  balance   - per-expert bias update from the batch's expert load
              (auxiliary-loss-free balancing; mastering-deepseek-v4, Implemented
              and Measured)

Parity pinned by tests/test_oracle_*.py; see each module's header for the pins
and for the functions whose parity the pages leave unpinned.
"""
