"""NTK-aware RoPE base scaling, float64 oracle (test infrastructure only).

The pages only name the method: "Llama2 Transformer架构解析与优化实践", section 6.1,
lists NTK-aware scaling beside linear interpolation as a way to extend RoPE
past the trained length, by adjusting the rotation angles, and gives no
formula.  The definition followed is the published one (the "NTK-aware scaled
RoPE" proposal of 2023, also the "dynamic NTK" rotary embedding of the
Hugging Face Transformers library): instead of dividing positions, raise the
base theta so that the highest frequency keeps its value and the lowest
frequency is divided by the scale alpha:

    theta' = theta * alpha ** (D / (D - 2))

so inv_freq'_i = theta'^(-2i/D) = inv_freq_i * alpha^(-2i/(D-2)): 1 at i = 0,
1/alpha at i = D/2 - 1.  The dynamic form picks alpha from the sequence
length L and the trained length L0 with a factor f: alpha = f * L / L0 - (f - 1)
when L > L0, and leaves theta unchanged otherwise.  Positions are not divided
(the linear factor stays 1); the rotation itself is the oracle's ``rope``.
"""
import numpy as np


def ntk_theta(theta, head_dim, alpha):
    """theta * alpha ** (D / (D - 2)), float64."""
    D = int(head_dim)
    if D < 4 or D % 2:
        raise ValueError("head_dim must be even and at least 4")
    if not (alpha > 0):
        raise ValueError("alpha must be positive")
    return np.float64(theta) * np.power(np.float64(alpha), np.float64(D) / np.float64(D - 2))


def dynamic_ntk_theta(theta, head_dim, factor, seq_len, max_position):
    """The dynamic form: alpha = factor * seq_len / max_position - (factor - 1)
    for sequences longer than max_position, else theta unchanged."""
    if seq_len <= max_position:
        return np.float64(theta)
    alpha = np.float64(factor) * np.float64(seq_len) / np.float64(max_position) - (np.float64(factor) - 1.0)
    return ntk_theta(theta, head_dim, alpha)
