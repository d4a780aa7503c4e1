"""CPU oracle for Introspective Strided Decoding (ISD) and its gated-LoRA variant R-ISD.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
package: only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP library
(``strided_decoding_amd``); the only module both sides use is ``isd_inputs``, which
draws seeded synthetic inputs and holds none of the method's arithmetic.

The oracle is a plain, slow, obviously-correct restatement of what the decode step
computes, written from the pages about the method:

* Bud's Wiki note "Introspective Diffusion Language Models", sections *TL;DR*,
  *Key claims* and *Method* (strict causal attention, logit shift, the
  min(1, p/q) acceptance rule, first-rejection restart, the TPF closed form,
  R-ISD gated LoRA);
* the Agentic Commons post of the same title, section *How Introspective Strided
  Decoding Works* (acceptance borrowed from speculative sampling, output
  distribution equal to the AR model's);
* the GeekNews summaries (Hindi and Portuguese), sections *Throughput*,
  *Speedup Factor Explorer*, *Inference & ISD*, *Serving (SGLang)* and
  *Lossless R-ISD*.

Modules
-------
philox   Philox4x32-10 counter-based generator (Salmon et al., SC'11) and the
         uniform u(slot, t, position, purpose) both sides draw.
model    fp32 pre-norm causal transformer with RoPE, GQA, SwiGLU and the
         MASK-row-gated LoRA; dense attention over a gathered KV cache.
sampler  softmax with temperature, categorical draw by inverse CDF, the
         acceptance test, the residual resample, argmax with lowest-index ties.
paged_kv LIFO page allocator and page tables.
isd      the ISD / R-ISD / AR decoders (per-slot A/B state machine).
tpf      tokens-per-forward closed form and a Monte-Carlo of the state machine.

Parity status of each function is stated in its docstring; every function here
is pinned by a test in ``tests/test_oracle_*.py`` except where the docstring says
"parity unpinned".
"""
