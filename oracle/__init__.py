"""CPU oracle of the denoising step (NumPy float64).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package. It shares no code with the HIP path; the
only module both sides use is the seeded input generator
(block_discrete_diffusion_dg_amd.synth), which holds no arithmetic of the step.

Parity status per function (what pins each, see tests/test_oracle_pins.py):
  philox4x32_10   published known-answer vectors (Salmon et al., SC'11)
  uniform_ids     chi-square uniformity; power-of-two shift identity
  rms_norm        closed form on constant rows; scale invariance
  rope            norm preservation; relative-position property; 2-D rotation
  attention       torch scaled_dot_product_attention (CPU, float64); rows of
                  softmax sum to 1; equal scores give the mean of V; causal
                  with empty prefix equals textbook causal attention
  route           numpy stable argsort; k = 1 and k = E special cases
  permutation     numpy stable argsort of the expert ids; bijection
  moe             k = E equals the dense softmax mixture of all experts
  row_stats       numpy argmax / scipy logsumexp
  sample          invariants (ids in range, |accepted| = k_s, held tokens kept
                  unless re-noised, last step accepts everything)
  whole step      zero-layer model reduces to RMSNorm(E[x]) E^T; causal
                  consistency of prefill vs prefill + commit
  row_entropy     closed forms (uniform, two tokens, k-way ties); scipy's
                  entropy of the softmax; temperature monotonicity
  adaptive_stop   its four cases; a stopped step accepts every position
  gumbel_candidates  chi-square against softmax(L / tau) over 20,000
                  positions; argmax at vanishing temperature; uniforms on
                  the 23-bit grid inside (0, 1), distinct streams
  fp8 (E4M3)      torch's float8_e4m3fn decode and encode; round trip of
                  every finite code; ties to even; row-exponent minimality;
                  half-ulp error bound
  ar_step         equals a causal pass over the whole sequence from an
                  empty cache (K/V rows, last-row logits, next token)
  metrics         the pages' worked TPF/TPS example
Fidelity to the trained DiffusionGemma model: parity unpinned (no weights).
"""
