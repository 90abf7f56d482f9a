"""Rotary position embedding, float64 oracle (test infrastructure only).

Definition followed (sources are the pages' titles and sections):

* Rotation applies to queries and keys only, after their projections; values
  are never rotated ("LLaMA2大语言模型架构详解", section "Rotary Position
  Encoding", the Tips list; "【HuggingFace Transformers】LlamaAttention源码解析",
  section 2, forward step 3).
* The rotation is RoFormer's (named in the same section of the LLaMA2 page):
  pair i of a head vector turns by the angle ``pos * theta**(-2 i / D)``,
  ``i = 0 .. D/2-1``, with base ``theta`` = the config's ``rope_theta``
  (LlamaAttention walkthrough, section 2, ``__init__``).
* The rotation is the complex-domain product of a pair with ``exp(i*angle)``
  ("Llama2 Transformer架构解析与优化实践", section 2.1); written as
  ``x*cos + rotate(x)*sin``.  Pairing (a reading -- the pages print neither
  ``apply_rotary_pos_emb`` nor ``rotate_half``): the default "half" pairing
  takes ``(x[i], x[i + D/2])``, ``rotate(x) = [-x2, x1]``; the "interleaved"
  pairing takes ``(x[2i], x[2i+1])``.
* Linear position scaling ("Llama2 Transformer架构解析与优化实践", section 6.1,
  ``rope_scaling = {type: linear, factor}``): positions are divided by the
  factor before the angle is formed; theta is left unchanged.
"""
import numpy as np


def inv_freq(head_dim, theta):
    """theta ** (-2 i / D) for i = 0 .. D/2 - 1, float64 (RoFormer frequencies)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(head_dim))


def angles(positions, head_dim, theta, linear_factor=1.0):
    """Angle of every pair: (pos / factor) * inv_freq, shape positions.shape + (D/2,)."""
    pos = np.asarray(positions, dtype=np.float64) / np.float64(linear_factor)
    return pos[..., None] * inv_freq(head_dim, theta)


def rotate(x, positions, theta, linear_factor=1.0, style="half"):
    """Rotate every head vector in ``x`` (shape [..., D]) by its position.

    ``positions`` broadcasts against ``x.shape[:-1]``.  Returns a new float64
    array; ``x`` is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = angles(positions, D, theta, linear_factor)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    if style == "half":
        x1, x2 = x[..., : D // 2], x[..., D // 2:]
        out[..., : D // 2] = x1 * c - x2 * s
        out[..., D // 2:] = x2 * c + x1 * s
    elif style == "interleaved":
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = x1 * c - x2 * s
        out[..., 1::2] = x2 * c + x1 * s
    else:
        raise ValueError(f"unknown rope style {style!r}")
    return out


def rope_apply(q, k, position_ids, theta, linear_factor=1.0, style="half"):
    """Rotate q [B,S,Hq,D] and k [B,S,Hkv,D] at position_ids [B,S].

    ``position_ids=None`` means 0..S-1 for every sequence (the default
    ``position_ids`` of the LlamaAttention walkthrough, section 2).
    Returns float64 copies (q_rot, k_rot).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, S = q.shape[0], q.shape[1]
    if position_ids is None:
        position_ids = np.broadcast_to(np.arange(S), (B, S))
    pos = np.asarray(position_ids)[:, :, None]  # broadcast over heads
    return (rotate(q, pos, theta, linear_factor, style),
            rotate(k, pos, theta, linear_factor, style))
