"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds workload presets (shapes only), the seeded generators, and the storage
encodings the inputs are handed over in.  None of the forward arithmetic lives
here.  The byte generators are C (``synth.c``, built into ``libsynth.so`` next
to this file); this module wraps them with numpy.

Workloads follow the Phi-3-mini-4k shape named on the page "Phi-3-mini:
fused-tensor direct loading in a sovereign inference engine" (section 2,
Methods: head_dim 96, untied lm_head; section 1: fused Q/K/V and gate/up
tensors), and the Phi-4 decode geometry of "Phi-4: quality transfer and
interrupted throughput studies" (setup paragraph: 40 query heads, 10 KV heads,
head_dim 128, FP16 keys, E4M3 values; pool paragraph: paged KV).
"""
from __future__ import annotations

import ctypes
import hashlib
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

WEIGHT_SEED = 1
IDS_SEED = 2
DECODE_SEED = 3
WEIGHT_STD = 0.02


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so with gcc (host code only)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread", src, "-o", tmp, "-lm"]
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # SYNTH_LIB names another build of synth.c (the host-sanitizer test uses it)
    path = os.environ.get("SYNTH_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path):
            build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    u64, i64, i32, dbl, cs = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_char_p
    for nm in ("synth_normal_f64", "synth_normal_f32", "synth_normal_f16"):
        getattr(lib, nm).argtypes = [u64, cs, dbl, i64, P, ctypes.c_int]
        getattr(lib, nm).restype = None
    lib.synth_uniform_i32.argtypes = [u64, cs, i64, i32, P]
    lib.synth_permutation.argtypes = [u64, cs, i32, P]
    lib.synth_encode_f16.argtypes = [P, i64, P]
    lib.synth_decode_f16.argtypes = [P, i64, P]
    lib.synth_encode_e4m3.argtypes = [P, i64, dbl, P]
    lib.synth_quantize_rows_i8.argtypes = [P, i64, i64, P, P, ctypes.c_int]
    lib.synth_f64_to_f16.argtypes = [dbl]
    lib.synth_f64_to_f16.restype = ctypes.c_uint16
    lib.synth_f64_to_e4m3.argtypes = [dbl]
    lib.synth_f64_to_e4m3.restype = ctypes.c_uint8
    lib.synth_fnv1a64.argtypes = [cs]
    lib.synth_fnv1a64.restype = u64
    _lib = lib
    return lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- generators
def normal(seed: int, name: str, shape, std: float = 1.0, dtype=np.float64) -> np.ndarray:
    """std * N(0,1) from the counter-based stream `name`, rounded to `dtype`
    (float64, float32, or float16 with round-to-nearest-even from double)."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    dtype = np.dtype(dtype)
    out = np.empty(n, dtype=dtype)
    fn = {np.dtype(np.float64): lib.synth_normal_f64, np.dtype(np.float32): lib.synth_normal_f32,
          np.dtype(np.float16): lib.synth_normal_f16}[dtype]
    fn(seed, name.encode(), float(std), n, _ptr(out), _threads())
    return out.reshape(shape)


def uniform_ints(seed: int, name: str, shape, high: int) -> np.ndarray:
    lib = _load()
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int32)
    lib.synth_uniform_i32(seed, name.encode(), n, int(high), _ptr(out))
    return out.reshape(shape)


def permutation(seed: int, name: str, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int32)
    lib.synth_permutation(seed, name.encode(), int(n), _ptr(out))
    return out


def to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to binary16 (RNE), as a float16 array."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.synth_encode_f16(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


def to_e4m3(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Encode x / scale as OCP E4M3FN bytes (RNE, saturating to +-448)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.synth_encode_e4m3(_ptr(x), x.size, float(scale), _ptr(out))
    return out


def quantize_rows_i8(w16: np.ndarray):
    """Symmetric per-output-row int8 of a binary16 weight [N, K]:
    returns (q int8 [N, K], scale float16 [N])."""
    lib = _load()
    w16 = np.ascontiguousarray(w16, dtype=np.float16)
    n, k = w16.shape
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty(n, dtype=np.uint16)
    lib.synth_quantize_rows_i8(_ptr(w16), n, k, _ptr(q), _ptr(s), _threads())
    return q, s.view(np.float16)


# ---------------------------------------------------------------- presets
@dataclass(frozen=True)
class PhiConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    max_pos: int = 4096
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    wtype: str = "f16"          # "f32", "f16" or "i8" (per-row int8 + f16 scale)
    norm_gain: str = "normal"   # "normal": N(0, 0.02) like every weight; "ones": diagnostic
    qkv_bias: bool = False      # a bias on the fused QKV product (Qwen2-style)
    tie_embeddings: bool = False  # lm_head is the embedding matrix

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def act_dtype(self):
        return np.float32 if self.wtype == "f32" else np.float16

    def linear_shapes(self):
        h, i = self.hidden, self.intermediate
        return {"qkv": (self.qkv_rows, h), "o": (h, self.n_heads * self.head_dim),
                "gate_up": (2 * i, h), "down": (h, i)}


TINY = PhiConfig("tiny", n_layers=2, hidden=384, n_heads=4, n_kv_heads=4, head_dim=96,
                 intermediate=1024, vocab=4096, wtype="f32")
MINI = PhiConfig("mini", n_layers=32, hidden=3072, n_heads=32, n_kv_heads=32, head_dim=96,
                 intermediate=8192, vocab=32064, wtype="f16")
MINI_W8 = replace(MINI, name="mini_w8", wtype="i8")
# grouped-query attention at head_dim 128 (the Phi-4 geometry): a small model
# for oracle pins and one layer at full Phi-4 width (hidden 5120, 40 query
# heads over 10 KV heads, intermediate 17920, RoPE base 250000)
TINY_GQA128 = PhiConfig("tiny_gqa128", n_layers=2, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128,
                        intermediate=1024, vocab=4096, rope_theta=250000.0, wtype="f16")
PHI4_1L = PhiConfig("phi4_1l", n_layers=1, hidden=5120, n_heads=40, n_kv_heads=10, head_dim=128,
                    intermediate=17920, vocab=100352, rope_theta=250000.0, wtype="f16")
# the two other dense families of the parity harness page, at their public
# shapes: Qwen2.5-0.5B-style (GQA 14/2 at head_dim 64, QKV bias, tied
# embeddings) and SmolLM2-360M-style (GQA 15/5 at head_dim 64, tied)
QWEN25_05B = PhiConfig("qwen25_05b", n_layers=24, hidden=896, n_heads=14, n_kv_heads=2, head_dim=64,
                       intermediate=4864, vocab=151936, rms_eps=1e-6, rope_theta=1000000.0, wtype="f16",
                       qkv_bias=True, tie_embeddings=True)
SMOLLM2_360M = PhiConfig("smollm2_360m", n_layers=32, hidden=960, n_heads=15, n_kv_heads=5, head_dim=64,
                         intermediate=2560, vocab=49152, rms_eps=1e-5, rope_theta=100000.0, wtype="f16",
                         tie_embeddings=True)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    cfg: PhiConfig
    batch: int
    seq: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seq


PREFILL_WORKLOADS = {
    "tiny_f32_1x16": PrefillWorkload("tiny_f32_1x16", TINY, 1, 16),
    "mini_f16_1x512": PrefillWorkload("mini_f16_1x512", MINI, 1, 512),
    "mini_f16_1x4096": PrefillWorkload("mini_f16_1x4096", MINI, 1, 4096),
    "mini_w8_4x1024": PrefillWorkload("mini_w8_4x1024", MINI_W8, 4, 1024),
}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    ctx: int
    n_q_heads: int = 40
    n_kv_heads: int = 10
    head_dim: int = 128
    page_size: int = 16

    @property
    def pages_per_seq(self) -> int:
        return -(-self.ctx // self.page_size)

    @property
    def n_pages(self) -> int:
        return self.batch * self.pages_per_seq


DECODE_WORKLOADS = {
    "decode_k16v8_32x1024": DecodeWorkload("decode_k16v8_32x1024", 32, 1024),
    "decode_k16v8_16x8192": DecodeWorkload("decode_k16v8_16x8192", 16, 8192),
}


# ---------------------------------------------------------------- prefill inputs
def token_ids(cfg: PhiConfig, batch: int, seq: int, seed: int = IDS_SEED) -> np.ndarray:
    """Uniform ids over [0, vocab), int32 [batch, seq].  No BOS is prepended,
    so position 0 holds the first drawn id.  Flat element b*seq + s, so a
    batch-1 input is a prefix of any longer batch-1 input."""
    return uniform_ints(seed, "ids", (batch, seq), cfg.vocab)


def _stored(cfg: PhiConfig, name: str, shape, seed: int):
    dt = np.float32 if cfg.wtype == "f32" else np.float16
    return normal(seed, name, shape, WEIGHT_STD, dt)


def _gain(cfg: PhiConfig, name: str, seed: int):
    if cfg.norm_gain == "ones":
        return np.ones(cfg.hidden, dtype=cfg.act_dtype)
    return _stored(cfg, name, (cfg.hidden,), seed)


def _linear(cfg: PhiConfig, name: str, shape, seed: int):
    w = _stored(cfg, name, shape, seed)
    if cfg.wtype == "i8":
        return quantize_rows_i8(w)
    return w


def layer_weights(cfg: PhiConfig, layer: int, seed: int = WEIGHT_SEED) -> dict:
    """Weights of one decoder layer, as stored: float32, float16, or for the
    int8 path (q int8 [N, K], scale float16 [N]) tuples quantized from the
    seeded float16 weights."""
    p = f"layers.{layer}."
    out = {"ln1": _gain(cfg, p + "ln1", seed), "ln2": _gain(cfg, p + "ln2", seed)}
    for nm, shape in cfg.linear_shapes().items():
        out[nm] = _linear(cfg, p + nm, shape, seed)
    if cfg.qkv_bias:
        # activation type (float16 also for int8 weights)
        out["qkv_bias"] = normal(seed, p + "qkv_bias", (cfg.qkv_rows,), WEIGHT_STD, cfg.act_dtype)
    return out


def embed_weight(cfg: PhiConfig, seed: int = WEIGHT_SEED):
    return _stored(cfg, "embed", (cfg.vocab, cfg.hidden), seed)


def final_norm_weight(cfg: PhiConfig, seed: int = WEIGHT_SEED):
    return _gain(cfg, "final_norm", seed)


def lm_head_weight(cfg: PhiConfig, seed: int = WEIGHT_SEED):
    if cfg.tie_embeddings:
        e = embed_weight(cfg, seed)
        return quantize_rows_i8(e) if cfg.wtype == "i8" else e
    return _linear(cfg, "lm_head", (cfg.vocab, cfg.hidden), seed)


def as_f16_config(cfg: PhiConfig) -> PhiConfig:
    """The float16 model the int8 weights were quantized from."""
    return replace(cfg, name=cfg.name + "_f16src", wtype="f16") if cfg.wtype == "i8" else cfg


class WeightSet:
    """All weights of a model, generated lazily and cached per tensor group."""

    def __init__(self, cfg: PhiConfig, seed: int = WEIGHT_SEED, cache_layers: bool = True):
        self.cfg, self.seed, self.cache_layers = cfg, seed, cache_layers
        self._layers: dict[int, dict] = {}
        self._embed = self._final = self._lm = None

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        w = layer_weights(self.cfg, l, self.seed)
        if self.cache_layers:
            self._layers[l] = w
        return w

    @property
    def embed(self):
        if self._embed is None:
            self._embed = embed_weight(self.cfg, self.seed)
        return self._embed

    @property
    def final_norm(self):
        if self._final is None:
            self._final = final_norm_weight(self.cfg, self.seed)
        return self._final

    @property
    def lm_head(self):
        if self.cfg.tie_embeddings and self.cfg.wtype != "i8":
            return self.embed          # the same array: a tied model shares the tensor
        if self._lm is None:
            self._lm = lm_head_weight(self.cfg, self.seed)
        return self._lm

    def digest(self) -> str:
        """SHA-256 over every stored weight byte, in a fixed order."""
        h = hashlib.sha256()

        def feed(a):
            if isinstance(a, tuple):
                for t in a:
                    feed(t)
            else:
                h.update(np.ascontiguousarray(a).tobytes())

        feed(self.embed)
        for l in range(self.cfg.n_layers):
            w = self.layer(l)
            for nm in ("ln1", "qkv", "o", "ln2", "gate_up", "down", "qkv_bias"):
                if nm in w:
                    feed(w[nm])
        feed(self.final_norm)
        feed(self.lm_head)
        return h.hexdigest()


# ---------------------------------------------------------------- decode inputs
@dataclass
class DecodeInputs:
    wl: DecodeWorkload
    q: np.ndarray            # float16 [B, Hq, D]
    k_pool: np.ndarray       # float16 [P, Hkv, page, D]
    v_pool: np.ndarray       # uint8 E4M3FN codes [P, Hkv, page, D]
    v_scale: np.ndarray      # float32 [Hkv]
    block_table: np.ndarray  # int32 [B, pages_per_seq]
    ctx_lens: np.ndarray     # int32 [B]
    extra: dict = field(default_factory=dict)


def decode_inputs(wl: DecodeWorkload, seed: int = DECODE_SEED, ctx_lens=None) -> DecodeInputs:
    """Q, K ~ N(0,1) in float16; V ~ N(0,1) stored as E4M3FN with one float32
    scale per KV head, amax(V_head) / 448; block table = a random permutation
    of all physical pages, so logical and physical page order differ."""
    B, Hq, Hkv, D, pg = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.page_size
    P = wl.n_pages
    q = normal(seed, "decode.q", (B, Hq, D), 1.0, np.float16)
    k = normal(seed, "decode.k", (P, Hkv, pg, D), 1.0, np.float16)
    v = normal(seed, "decode.v", (P, Hkv, pg, D), 1.0, np.float64)
    amax = np.abs(v).max(axis=(0, 2, 3))
    scale = (amax / 448.0).astype(np.float32)
    vb = to_e4m3(v / scale.astype(np.float64)[None, :, None, None], 1.0)
    del v
    bt = permutation(seed, "decode.pages", P).reshape(B, wl.pages_per_seq)
    if ctx_lens is None:
        ctx_lens = np.full(B, wl.ctx, dtype=np.int32)
    return DecodeInputs(wl, q, k, vb, scale, bt, np.asarray(ctx_lens, dtype=np.int32))
