"""Storage accounting for NF4 + double quantisation and for LoRA adapters.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

These are the plain counting formulas behind the worked numbers the pages
print; ``tests/golden/page_worked_examples.json`` holds those numbers with
their citations and ``tests/test_oracle_memory.py`` checks the formulas
against them.
"""


def bits_per_param(blocksize=64, group=256, double_quant=True, code_bits=4):
    """Storage bits per weight: the code plus its share of the constants.

    Without double quantisation each block of ``blocksize`` weights carries
    one fp32 constant ([rkmt] §2.2.2).  With it, each block carries an 8-bit
    code and each group of ``group`` blocks one fp32 constant (reading of
    [rkmt] §2.2.2 and [kwkr] §3.1).
    """
    if double_quant:
        return code_bits + 8.0 / blocksize + 32.0 / (blocksize * group)
    return code_bits + 32.0 / blocksize


def dq_saving_bits(blocksize=64, group=256):
    """Bits per weight saved by double quantisation ([tgd] §2, [kwkr] §3.1)."""
    return (bits_per_param(blocksize, group, False)
            - bits_per_param(blocksize, group, True))


def constant_bytes(n_params, blocksize=64, group=256, double_quant=True):
    """Bytes of quantisation constants for ``n_params`` weights."""
    nblocks = -(-n_params // blocksize)
    if not double_quant:
        return 4 * nblocks
    return nblocks + 4 * (-(-nblocks // group))


def dq_constant_bytes_single_global(nblocks):
    """[rkmt] §2.2.2's own count: N one-byte codes plus two fp32 globals."""
    return nblocks * 1 + 2 * 4


def quantized_weight_bytes(n_params, blocksize=64, group=256, double_quant=True):
    """Packed 4-bit codes plus constants, in bytes."""
    return n_params // 2 + constant_bytes(n_params, blocksize, group, double_quant)


def dense_bytes(n_params, bytes_per_param=2):
    """Unquantised storage (fp16/bf16 by default)."""
    return n_params * bytes_per_param


def lora_params(shapes, r):
    """Trainable LoRA parameters: r (N + K) for every adapted N x K matrix."""
    return sum(r * (n + k) for (n, k) in shapes)


def llama7b_target_shapes(hidden=4096, mlp=11008, layers=32):
    """The seven adapted projections of a Llama-7B-shaped decoder, all layers.

    q, k, v, o: hidden x hidden; gate, up: mlp x hidden; down: hidden x mlp
    ([tgd] §4 and [rkmt] §3.3 list these seven target modules).
    """
    per_layer = [(hidden, hidden)] * 4 + [(mlp, hidden)] * 2 + [(hidden, mlp)]
    return per_layer * layers
