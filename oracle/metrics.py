"""Throughput metrics of the pages (test infrastructure; never used by the product path).

codemajin.net DiffusionGemma explainer, §5.1:
  TPF = generated tokens / (denoising steps + K - 1), K = number of blocks
        (each committed block costs one extra forward to append it to the
        KV cache, except the last);
  TPS = TPF / t_fwd, t_fwd = wall time of one denoising forward.
"""


def tokens_per_forward(generated_tokens: int, denoise_steps: int, blocks: int) -> float:
    return generated_tokens / (denoise_steps + blocks - 1)


def tokens_per_second(tpf: float, t_fwd_seconds: float) -> float:
    return tpf / t_fwd_seconds
