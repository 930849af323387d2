"""The synthetic workloads: five configurations of seeded payloads.

Shapes, value ranges and formats follow the benchmark configurations of this
project (LLM weight matrices); seeds are fixed so every run, test and
benchmark sees the same bytes.  Each tensor is (name, format, shape, recipe,
seed).  Block size B is not known here: callers take it from the registry.

  1  q8_0 and q4_0 [64, 4096] -> f32; binary16 scales |d| in [2^-12, 2^-6),
     random sign; codes uniform bytes.
  2  q4_k and q6_k [4096, 4096] -> bf16; d, dmin positive in [2^-14, 2^-8);
     packed sub-scales, mins and codes uniform bytes.
  3  mxfp4 (E8M0 byte in [118, 130]) and nvfp4 (E4M3FN scale bytes in
     [0x01, 0x7E], divisor bits uniform in [bits(1.0), bits(448.0)])
     [14336, 4096] -> bf16.
  4  iq2_xxs, iq2_s, iq3_s, iq1_m, iq4_nl, iq4_xs [4096, 14336] -> f32 and
     bf16; d positive in [2^-12, 2^-6); every other byte uniform (all index,
     sign and sub-scale fields legal at every value).
  5  A Llama-3-8B-shaped weight set, 226 tensors: embedding, then per layer
     wq, wk, wv, wo, w_gate, w_up, w_down, then lm_head; tensor t uses
     [q4_k, q6_k, q8_0, nvfp4, tq2_0][t mod 5] with the ranges above (tq2_0:
     d positive in [2^-12, 2^-6), codes uniform in {0, 1, 2}); all -> bf16.
"""
from . import binade

SEED_BASE = 0x6E710000


def seed(config, format_index, tensor=0):
    return SEED_BASE + 1_000_000 * tensor + 1000 * config + 10 * format_index


def recipe_for(fmt):
    """Scale-field recipe of a format in these workloads."""
    if fmt in ("gguf:q4_k", "gguf:q6_k"):
        return binade(-14, -8, False)
    if fmt in ("gguf:q8_0", "gguf:q4_0"):
        return binade(-12, -6, True)
    return binade(-12, -6, False)


def config1():
    return [(f"cfg1.{f[5:]}", f, [64, 4096], recipe_for(f), seed(1, i))
            for i, f in enumerate(["gguf:q8_0", "gguf:q4_0"])], ["f32"]


def config2():
    return [(f"cfg2.{f[5:]}", f, [4096, 4096], recipe_for(f), seed(2, i))
            for i, f in enumerate(["gguf:q4_k", "gguf:q6_k"])], ["bf16"]


def config3():
    return [(f"cfg3.{f.split(':')[-1]}", f, [14336, 4096], recipe_for(f), seed(3, i))
            for i, f in enumerate(["gguf:mxfp4", "nvfp4"])], ["bf16"]


CONFIG4_FORMATS = ["gguf:iq2_xxs", "gguf:iq2_s", "gguf:iq3_s", "gguf:iq1_m", "gguf:iq4_nl", "gguf:iq4_xs"]


def config4():
    return [(f"cfg4.{f[5:]}", f, [4096, 14336], recipe_for(f), seed(4, i))
            for i, f in enumerate(CONFIG4_FORMATS)], ["f32", "bf16"]


CONFIG5_ROTATION = ["gguf:q4_k", "gguf:q6_k", "gguf:q8_0", "nvfp4", "gguf:tq2_0"]
LLAMA3_8B_LAYER = [("wq", [4096, 4096]), ("wk", [1024, 4096]), ("wv", [1024, 4096]), ("wo", [4096, 4096]),
                   ("w_gate", [14336, 4096]), ("w_up", [14336, 4096]), ("w_down", [4096, 14336])]


def config5_shapes():
    out = [("embedding", [128256, 4096])]
    for layer in range(32):
        out += [(f"layers.{layer}.{n}", s) for n, s in LLAMA3_8B_LAYER]
    out.append(("lm_head", [128256, 4096]))
    return out


def config5():
    tensors = []
    for t, (name, shape) in enumerate(config5_shapes()):
        f = CONFIG5_ROTATION[t % 5]
        tensors.append((f"cfg5.{name}", f, shape, recipe_for(f), seed(5, CONFIG5_ROTATION.index(f), t)))
    return tensors, ["bf16"]


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
