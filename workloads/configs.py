"""The five benchmark workloads plus small parity cases.

Shapes follow the pages' settings: a Llama-3.1-8B-like GQA attention shape (32 query
heads sharing 8 KV heads of width 128) as evaluated by LogQuant (page
"LogQuant: Log-Distributed 2-Bit Quantization of KV Cache", experimental results) and
by AATC (page "KV Cache Compression Through the Lens of Transform Coding", results);
K4V2 bit allocation ("Quantize What Counts: More for Keys, Less for Values",
methodology and results); log-spaced full-precision retention (LogQuant, log-based
filtering strategy); thin keys with d_select = d_model/4 ("Thin Keys, Full Values",
asymmetric attention).
"""

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    T: int
    k_bits: int
    v_bits: int
    n_recent: int = 0        # newest tokens kept in fp16
    log_window: int = 0      # W of the log-spaced fp16 regions (0 = off)
    dtype: str = "bf16"      # dtype of q, K and V as handed to both sides: "f32" | "bf16" | "f16"
    partitions: int = 1      # split-K sequence partitions used by decode
    seed: int = 0
    prefill_chunk: int = 0   # tokens of the newest chunk re-packed inside one bench step
    key_rotation: bool = False  # keys rotated (Walsh-Hadamard) before quantization
    k_group: int = 32
    v_group: int = 32
    n_outliers: int = 4
    outlier_scale: float = 8.0
    k_offset_std: float = 2.0
    v_std: float = 0.5
    notes: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny_ref", B=1, Hq=1, Hkv=1, Dk=64, Dv=64, T=256, k_bits=4, v_bits=2,
             dtype="f32", partitions=1, seed=0,
             notes="one fp32 query, no fp16 window"),
    Workload("llama8b_gqa_4k", B=8, Hq=32, Hkv=8, Dk=128, Dv=128, T=4096, k_bits=4, v_bits=2,
             n_recent=128, dtype="bf16", partitions=4, seed=1,
             notes="K4V2, newest 128 tokens fp16"),
    Workload("logquant_32k", B=32, Hq=32, Hkv=8, Dk=128, Dv=128, T=32768, k_bits=2, v_bits=2,
             n_recent=128, log_window=128, dtype="bf16", partitions=16, seed=2,
             notes="K2V2, 128 fp16 window + log-spaced fp16 tokens (640 kept)"),
    Workload("thin_keys_16k", B=16, Hq=32, Hkv=8, Dk=32, Dv=128, T=16384, k_bits=8, v_bits=4,
             dtype="bf16", partitions=8, seed=3,
             notes="d_select = 32 keys, full 128-wide values, K8V4"),
    Workload("long_128k", B=4, Hq=32, Hkv=8, Dk=128, Dv=128, T=131072, k_bits=4, v_bits=2,
             n_recent=128, dtype="bf16", partitions=64, seed=4, prefill_chunk=8192,
             notes="K4V2, 128 fp16 window, 64 split-K partitions, 8192-token prefill chunk"),
]


def workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


def small_cases():
    """Shapes the oracle finishes in well under a second that still cover several
    groups, several partitions, uneven partition sizes and every bit width."""
    return [
        Workload("small_k4v2_win", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", partitions=5, seed=11),
        Workload("small_k2v2_log", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=2048, k_bits=2, v_bits=2,
                 n_recent=64, log_window=64, dtype="bf16", partitions=7, seed=12),
        Workload("small_k8v4_thin", B=2, Hq=8, Hkv=2, Dk=32, Dv=128, T=800, k_bits=8, v_bits=4,
                 dtype="bf16", partitions=3, seed=13),
        Workload("small_k4v8_f32", B=1, Hq=2, Hkv=1, Dk=64, Dv=96, T=352, k_bits=4, v_bits=8,
                 n_recent=32, dtype="f32", partitions=4, seed=14),
        Workload("small_g8_k2v4", B=1, Hq=16, Hkv=2, Dk=96, Dv=64, T=579, k_bits=2, v_bits=4,
                 n_recent=0, log_window=32, dtype="bf16", partitions=2, seed=15),
        # value groups wider than 32 channels (matrix-core and generic paths)
        Workload("small_k4v2_vg64", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", partitions=5, seed=16, v_group=64),
        Workload("small_k2v4_vg128_log", B=1, Hq=4, Hkv=1, Dk=128, Dv=128, T=1487, k_bits=2, v_bits=4,
                 n_recent=64, log_window=64, dtype="bf16", partitions=3, seed=17, v_group=128),
        Workload("small_g2_k8v8_vg64", B=1, Hq=4, Hkv=2, Dk=64, Dv=64, T=352, k_bits=8, v_bits=8,
                 n_recent=32, dtype="f32", partitions=4, seed=18, v_group=64),
        Workload("small_d256_k4v4_vg128", B=1, Hq=2, Hkv=2, Dk=256, Dv=256, T=288, k_bits=4, v_bits=4,
                 dtype="bf16", partitions=2, seed=19, v_group=128),
        # key groups longer than 32 tokens (matrix-core and generic paths, log-spaced fp16 tokens)
        Workload("small_k4v2_kg128", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", partitions=5, seed=20, k_group=128),
        Workload("small_k2v2_kg64_log", B=1, Hq=4, Hkv=1, Dk=128, Dv=128, T=1487, k_bits=2, v_bits=2,
                 n_recent=64, log_window=64, dtype="bf16", partitions=3, seed=21, k_group=64, v_group=64),
        Workload("small_g2_k8v4_kg64_f32", B=1, Hq=4, Hkv=2, Dk=96, Dv=64, T=416, k_bits=8, v_bits=4,
                 n_recent=32, dtype="f32", partitions=4, seed=22, k_group=64),
        # 3-bit codes (bit streams, codes straddle words; vector-ALU decode kernel)
        Workload("small_k3v3", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=3, v_bits=3,
                 n_recent=40, dtype="bf16", partitions=5, seed=26),
        Workload("small_k3v2_kg64_log", B=1, Hq=4, Hkv=1, Dk=96, Dv=128, T=1487, k_bits=3, v_bits=2,
                 n_recent=64, log_window=64, dtype="bf16", partitions=3, seed=27, k_group=64),
        Workload("small_g2_k4v3_vg64_f32", B=1, Hq=4, Hkv=2, Dk=64, Dv=64, T=352, k_bits=4, v_bits=3,
                 n_recent=32, dtype="f32", partitions=4, seed=28, v_group=64),
        # 1-bit codes (vector-ALU decode kernel)
        Workload("small_k1v1", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=544, k_bits=1, v_bits=1,
                 n_recent=32, dtype="bf16", partitions=3, seed=23),
        Workload("small_k4v1_log_vg64", B=1, Hq=4, Hkv=1, Dk=64, Dv=64, T=1487, k_bits=4, v_bits=1,
                 n_recent=64, log_window=64, dtype="bf16", partitions=2, seed=24, v_group=64),
        Workload("small_k1v4_f32", B=1, Hq=2, Hkv=1, Dk=32, Dv=96, T=352, k_bits=1, v_bits=4,
                 n_recent=32, dtype="f32", partitions=4, seed=25),
        # fp16 keys, values and queries (matrix-core and vector-ALU paths)
        Workload("small_k4v2_f16", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="f16", partitions=5, seed=29),
        Workload("small_g2_k4v4_f16_log", B=1, Hq=4, Hkv=2, Dk=64, Dv=96, T=579, k_bits=4, v_bits=4,
                 n_recent=0, log_window=32, dtype="f16", partitions=3, seed=30),
        # keys rotated before quantization (every pack and decode path: 128-wide and
        # generic pack, key groups of 64 tokens, retained rows, both decode kernels)
        Workload("small_k4v2_rot", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", partitions=5, seed=31, key_rotation=True),
        Workload("small_k2v2_log_rot_f16", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=2048, k_bits=2, v_bits=2,
                 n_recent=64, log_window=64, dtype="f16", partitions=7, seed=32, key_rotation=True),
        Workload("small_k8v4_thin_rot", B=2, Hq=8, Hkv=2, Dk=32, Dv=128, T=800, k_bits=8, v_bits=4,
                 n_recent=32, dtype="bf16", partitions=3, seed=33, key_rotation=True),
        Workload("small_k4v4_d64_rot_log", B=1, Hq=8, Hkv=2, Dk=64, Dv=128, T=1431, k_bits=4, v_bits=4,
                 n_recent=32, log_window=32, dtype="bf16", partitions=3, seed=34, key_rotation=True),
        Workload("small_g2_k8v4_kg64_rot_f32", B=1, Hq=4, Hkv=2, Dk=64, Dv=64, T=416, k_bits=8, v_bits=4,
                 n_recent=32, dtype="f32", partitions=4, seed=35, k_group=64, key_rotation=True),
        Workload("small_d256_k4v4_rot", B=1, Hq=2, Hkv=2, Dk=256, Dv=256, T=320, k_bits=4, v_bits=4,
                 n_recent=32, dtype="bf16", partitions=2, seed=36, v_group=128, key_rotation=True),
        Workload("small_k4v2_kg128_rot", B=1, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", partitions=5, seed=37, k_group=128, key_rotation=True),
    ]
