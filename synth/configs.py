"""Model shapes and workloads of the decode-step benchmarks (synthetic, seeded)."""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    tied: bool
    rope_theta: float
    eps: float = 1e-5
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0

    def with_(self, **kw):
        return replace(self, **kw)

    def weight_bytes(self):
        """bf16 bytes of every weight read by one decode step of one token (dense)."""
        h, d = self.hidden, self.head_dim
        per_layer = h * (self.n_q + 2 * self.n_kv) * d + self.n_q * d * h + 3 * h * self.ffn
        return 2 * (self.n_layers * per_layer + self.vocab * h) + 2 * (2 * self.n_layers + 1) * h


# Tiny Llama-style decoder: 2 layers, hidden 256, 4 Q / 2 KV heads of 64, SwiGLU 1024, vocab 4096.
TINY = ModelConfig("tiny", 2, 256, 4, 2, 64, 1024, 4096, True, 10000.0)
# Llama-3.2-1B shape: 16 layers, hidden 2048, 32 Q / 8 KV heads of 64, SwiGLU 8192, vocab 128256, tied.
LLAMA_1B = ModelConfig("llama-3.2-1b-shape", 16, 2048, 32, 8, 64, 8192, 128256, True, 500000.0)
# Llama-3-8B shape: 32 layers, hidden 4096, 32 Q / 8 KV heads of 128, SwiGLU 14336, vocab 128256, untied.
LLAMA_8B = ModelConfig("llama-3-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, False, 500000.0)
# Sparse MoE: 1B attention shape, 64 experts of SwiGLU 1024, top-8 routing.
MOE_1B = ModelConfig("moe-16l-64e-top8", 16, 2048, 32, 8, 64, 0, 128256, True, 500000.0,
                     n_experts=64, top_k=8, expert_ffn=1024)

# Tiny sparse MoE for the GPU tests: the tiny attention shape, 8 experts of SwiGLU 256, top-2.
TINY_MOE = ModelConfig("tiny-moe", 2, 256, 4, 2, 64, 0, 4096, True, 10000.0, n_experts=8, top_k=2, expert_ffn=256)

# Small dense decoder within the prompt megakernel's shape limits (hidden a multiple of 512, head_dim 64):
# 2 layers, hidden 512, 8 Q / 2 KV heads of 64, SwiGLU 1024, vocab 4096.
TINY_PF = ModelConfig("tiny-prompt", 2, 512, 8, 2, 64, 1024, 4096, True, 10000.0)

CONFIGS = {c.name: c for c in (TINY, LLAMA_1B, LLAMA_8B, MOE_1B, TINY_MOE, TINY_PF)}
