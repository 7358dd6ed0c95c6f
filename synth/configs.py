"""The five synthetic workloads, named by what they are, with their seeds.

* ``single_1024``: one 1024 x 1024 BF16 matrix, N(0, 0.02); x N(0, 1).
* ``qwen3_4b_layers``: 36 decoder layers of Qwen3-4B-shaped batch-1 GEMVs
  (q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728),
  weights N(0, 1/sqrt(K)) per matrix, one activation per matrix.
* ``odd_shapes``: 7x513, 1000x3001, 4097x1, 3x65536, each Gaussian N(0, 0.02)
  and heavy-tailed 0.02*t3, with injected rare values; plus every BF16 pattern.
* ``tied_embedding``: 151936 x 2560 N(0, 0.02) shared by gather and lm_head;
  4096 uniform token ids; and an fp8 e4m3 copy of the 1024 x 1024 matrix.
* ``qwen25_7b_step``: 28 Qwen2.5-7B-shaped layers plus a 152064 x 3584 lm_head,
  all N(0, 1/sqrt(K)).

The matrices of the layer sets, the step and the embedding table are drawn
with ``synth.blocked_normal_bf16`` (256-row blocks, one PCG64 stream per block);
the 1024 x 1024 matrix, the odd shapes and every activation with numpy's
``default_rng(seed)`` over the whole array.
"""
from __future__ import annotations

import math

QWEN3_4B = (("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
            ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728))
QWEN3_4B_LAYERS = 36

QWEN25_7B = (("q", 3584, 3584), ("k", 512, 3584), ("v", 512, 3584), ("o", 3584, 3584),
             ("gate", 18944, 3584), ("up", 18944, 3584), ("down", 3584, 18944))
QWEN25_7B_LAYERS = 28
QWEN25_7B_VOCAB = 152064
QWEN25_7B_HIDDEN = 3584

EMBED_VOCAB = 151936
EMBED_HIDDEN = 2560
N_IDS = 4096

ODD_SHAPES = ((7, 513), (1000, 3001), (4097, 1), (3, 65536))

SINGLE = dict(n=1024, k=1024, sigma=0.02, w_seed=1, x_seed=2)
EMBED = dict(w_seed=400000, ids_seed=400001, x_seed=400002)


def sigma_for(k: int) -> float:
    """1/sqrt(K) computed in float64 (the caller rounds it to fp32)."""
    return 1.0 / math.sqrt(k)


def qwen3_seed(layer: int, idx: int) -> tuple[int, int]:
    """(weight seed, activation seed) of matrix ``idx`` (q=0 .. down=6) in ``layer``."""
    return 100000 + 10 * layer + idx, 200000 + 10 * layer + idx


def qwen25_seed(layer: int, idx: int) -> int:
    return 500000 + 10 * layer + idx


QWEN25_LM_HEAD_SEED = 500999
QWEN25_X_SEED = 501000


def qwen25_x_seed(layer: int, idx: int) -> int:
    """Activation seed of matrix ``idx`` of ``layer`` when it is checked on its own (lm_head: idx 99, layer 0)."""
    return 600000 + 10 * layer + idx


def qwen3_matrices(layers: int = QWEN3_4B_LAYERS):
    """Every matrix of the Qwen3-4B layer set, in layer order: dicts of name, layer, n, k, sigma, seeds."""
    for layer in range(layers):
        for idx, (name, n, k) in enumerate(QWEN3_4B):
            ws, xs = qwen3_seed(layer, idx)
            yield dict(label=f"qwen3_4b.L{layer}.{name}", name=name, layer=layer, n=n, k=k, sigma=sigma_for(k),
                       w_seed=ws, x_seed=xs)


def qwen25_matrices(layers: int = QWEN25_7B_LAYERS, lm_head: bool = True):
    """Every matrix of the Qwen2.5-7B step (layers, then the lm_head)."""
    for layer in range(layers):
        for idx, (name, n, k) in enumerate(QWEN25_7B):
            yield dict(label=f"qwen25_7b.L{layer}.{name}", name=name, layer=layer, n=n, k=k, sigma=sigma_for(k),
                       w_seed=qwen25_seed(layer, idx), x_seed=qwen25_x_seed(layer, idx))
    if lm_head:
        yield dict(label="qwen25_7b.lm_head", name="lm_head", layer=layers, n=QWEN25_7B_VOCAB, k=QWEN25_7B_HIDDEN,
                   sigma=sigma_for(QWEN25_7B_HIDDEN), w_seed=QWEN25_LM_HEAD_SEED, x_seed=qwen25_x_seed(0, 99))


def embedding_matrix():
    """The tied embedding / lm_head table of the embedding workload."""
    return dict(label="tied_embedding", name="embed", layer=0, n=EMBED_VOCAB, k=EMBED_HIDDEN, sigma=0.02,
                w_seed=EMBED["w_seed"], x_seed=EMBED["x_seed"])


def odd_seed(index: int) -> int:
    return 300000 + index
