"""The five synthetic workloads the layer is checked and measured on.

Shapes follow the Qwen3-VL family (2B and 8B text towers) and a 32B
prompt-encoder shape with 64 query heads; all use plain-weight RMSNorm,
per-head q/k RMSNorm before the rotation, interleaved three-axis MRoPE with
split-half rotation, causal GQA attention and a SwiGLU FFN.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    seq_len: int
    n_layers: int = 1
    eps: float = 1e-6
    theta: float = 5e6
    sections: tuple = (24, 20, 20)
    dtype: str = "bf16"          # storage/operand type of weights and activations
    positions: str = "text"      # "text" or "image_span"
    seed: int = 0
    # image span (positions == "image_span"): first token, merged grid size
    span_start: int = 0
    span_h: int = 0
    span_w: int = 0
    deepstack_std: float = 0.0   # > 0: a DeepStack slab is added on the span rows
    extra: dict = field(default_factory=dict)

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def span_len(self):
        return self.span_h * self.span_w

    def gemm_flops(self, seq_len=None):
        """Algorithmic FLOPs of the four projections of one layer (2 per MAC)."""
        s = self.seq_len if seq_len is None else seq_len
        h, f = self.hidden, self.ffn
        return 2 * s * (h * (self.q_dim + 2 * self.kv_dim) + self.q_dim * h + 2 * h * f + f * h)

    def attn_flops(self, seq_len=None):
        """Causal attention FLOPs of one layer: QK^T and PV over the pairs j <= s."""
        s = self.seq_len if seq_len is None else seq_len
        return 2 * self.head_dim * s * (s + 1) * self.n_heads

    def layer_flops(self, seq_len=None):
        return self.gemm_flops(seq_len) + self.attn_flops(seq_len)

    def with_seq(self, seq_len, n_layers=None):
        """The same layer shape at another sequence length (text-only positions)."""
        d = dict(self.__dict__)
        d.update(seq_len=seq_len, positions="text", deepstack_std=0.0,
                 span_start=0, span_h=0, span_w=0,
                 n_layers=self.n_layers if n_layers is None else n_layers,
                 name=f"{self.name}@S{seq_len}")
        return LayerConfig(**d)


CONFIGS = {
    "tiny_f32": LayerConfig(
        name="tiny_f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
        seq_len=32, theta=1e6, sections=(12, 10, 10), dtype="f32"),
    "qwen3vl_2b_text": LayerConfig(
        name="qwen3vl_2b_text", hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128,
        ffn=6144, seq_len=1024),
    "qwen3vl_2b_image": LayerConfig(
        name="qwen3vl_2b_image", hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128,
        ffn=6144, seq_len=2048, positions="image_span", span_start=100, span_h=32,
        span_w=32, deepstack_std=0.5),
    "qwen3vl_8b_stack4": LayerConfig(
        name="qwen3vl_8b_stack4", hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
        ffn=12288, seq_len=4096, n_layers=4),
    "qwen3_32b_encoder": LayerConfig(
        name="qwen3_32b_encoder", hidden=5120, n_heads=64, n_kv_heads=8, head_dim=128,
        ffn=25600, seq_len=8192),
}


def get_config(name):
    return CONFIGS[name]
