"""Segment (layer) tables of the synthetic workloads.

Adasum is applied per layer, so every workload is a list of parameter
tensors flattened into one buffer with CSR offsets.  The lists follow the
parameter order of the standard model definitions.
"""

import numpy as np

# id -> (K workers, dtype name, description)
CONFIGS = {
    1: (2, "f32", "K=2 fp32, 4 segments 1000/4096/65536/262144, N(0,1)"),
    2: (8, "f32", "K=8 fp32, ResNet-50 tensor list, shared + independent N(0,1), cosine ~0.5"),
    3: (16, "f32", "K=16 fp32, BERT-Large tensor list, N(0, std 1e-3)"),
    4: (64, "f16", "K=64 fp16, BERT-Base tensor list, per-segment scale log-uniform in [1e-6, 1]"),
    5: (32, "bf16", "K=32 bf16, 20000 log-uniform segments in [1, 1e6], per-segment cosine U[-1,1], 5% zero segments"),
}


def resnet50_lengths():
    """ResNet-50 parameter tensors: conv1 + BN, 16 bottlenecks, fc.

    Each bottleneck holds a 1x1 (cin->w), 3x3 (w->w) and 1x1 (w->4w)
    convolution, each followed by a BatchNorm (weight, bias); the first block
    of a stage adds a 1x1 projection cin->4w with its BatchNorm.
    161 tensors, 25,557,032 parameters.
    """
    lengths = [64 * 3 * 7 * 7, 64, 64]
    cin = 64
    for width, blocks in ((64, 3), (128, 4), (256, 6), (512, 3)):
        for b in range(blocks):
            lengths += [cin * width, width, width]
            lengths += [width * width * 9, width, width]
            lengths += [width * 4 * width, 4 * width, 4 * width]
            if b == 0:
                lengths += [cin * 4 * width, 4 * width, 4 * width]
            cin = 4 * width
    lengths += [2048 * 1000, 1000]
    return lengths


def bert_lengths(hidden, ffn, layers, vocab=30522, max_pos=512, type_vocab=2):
    """BERT parameter tensors: embeddings, encoder layers, pooler.

    Embeddings: word (vocab x H), position (512 x H), token type (2 x H),
    LayerNorm (weight, bias).  Per layer: query, key, value and attention
    output (H x H + H each), LayerNorm, FFN in (H x F + F), FFN out
    (F x H + H), LayerNorm.  Pooler: H x H + H.
    BERT-Large (1024, 4096, 24): 391 tensors, 335,141,888 parameters.
    BERT-Base (768, 3072, 12): 199 tensors, 109,482,240 parameters.
    """
    h, f = hidden, ffn
    lengths = [vocab * h, max_pos * h, type_vocab * h, h, h]
    for _ in range(layers):
        for _qkvo in range(4):
            lengths += [h * h, h]
        lengths += [h, h]
        lengths += [h * f, f]
        lengths += [f * h, h]
        lengths += [h, h]
    lengths += [h * h, h]
    return lengths


def stress_lengths(nseg, seed):
    """Segment lengths max(1, floor(exp(U * ln 1e6))), U ~ U[0, 1)."""
    rng = np.random.default_rng(np.random.SeedSequence([5, seed, 0]))
    u = rng.random(nseg)
    return np.maximum(1, np.floor(np.exp(u * np.log(1e6)))).astype(np.int64)


def offsets_from_lengths(lengths):
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def config_offsets(config, seed=None):
    """CSR segment offsets of workload ``config`` (seed only matters for 5)."""
    if config == 1:
        lengths = [1000, 4096, 65536, 262144]
    elif config == 2:
        lengths = resnet50_lengths()
    elif config == 3:
        lengths = bert_lengths(1024, 4096, 24)
    elif config == 4:
        lengths = bert_lengths(768, 3072, 12)
    elif config == 5:
        lengths = stress_lengths(20000, 5 if seed is None else seed)
    else:
        raise ValueError(f"unknown workload {config}")
    return offsets_from_lengths(lengths)
