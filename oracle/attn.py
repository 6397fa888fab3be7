"""Oracle for the decode-time attention read of a 4-bit quantized K/V cache.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source passages: page 3 ("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"),
the architecture paragraph (64 layers in a repeating pattern of three
recurrent layers and one full-attention layer, so 16 layers keep a
conventional KV cache, held with 4-bit K and V at roughly 4.25 GiB for a
256K context) and the bandwidth paragraph (the 16 attention layers add K/V
reads that grow with the context, which takes the same model from about
50 tok/s to 12.61 tok/s at a 261.5K-token cache).  The pages give neither
the head geometry nor the cache layout.  Readings used here:

  * Layout: per layer, K and V are each a token-major matrix [T, H_kv * D]
    in the same 4-bit block format as the weights (32-element blocks along
    the head dimension, an fp16 scale absmax / 7, signed codes two per
    byte): codes [T, H_kv * D / 2] and scales [T, H_kv * D / 32], exactly
    what quantizing the fp32 rows of K (or V) with the weight quantizer
    gives.  A block never straddles two heads (D % 32 == 0).
  * Geometry (a reading, stated in the design notes): H_kv * D = 1024 per
    layer with D = 256, H_kv = 4 and H_q = 20 query heads (G = 5 query heads
    share one K/V head).  The functions here take any H_q, H_kv and D with
    H_q % H_kv == 0.
  * The M query tokens of a step (the target token and its drafted tokens)
    are the last M positions of the cache: query m sees positions
    0 .. T - M + m (causal among the drafts).
  * Scores q . k / sqrt(D); softmax over the visible positions; output the
    softmax-weighted sum of the V rows.  Query head h reads K/V head h // G.
  * Everything in float64 here, with the exact dequantized cache; the GPU
    dequantizes to fp16, accumulates in fp32 and returns fp16.
"""

import numpy as np

from . import q4


def dequantize_cache(codes, scales, n_heads):
    """Exact float64 cache [T, n_heads, D] from codes [T, H*D/2] and scales [T, H*D/32]."""
    w = q4.dequantize(q4.unpack(codes), scales)
    t, hd = w.shape
    if hd % n_heads:
        raise ValueError("row width is not a multiple of the head count")
    return w.reshape(t, n_heads, hd // n_heads)


def visible_length(t, m_count, m):
    """Positions query m of the last m_count tokens of a t-token cache sees."""
    return t - m_count + m + 1


def attention_decode(q, k_codes, k_scales, v_codes, v_scales, n_kv_heads):
    """o[m, h, :] = sum_t softmax_t(q[m, h] . K[t, g] / sqrt(D)) V[t, g], g = h // G.

    q is fp16 [M, H_q, D]; the caches follow the layout above; returns
    float64 [M, H_q, D].
    """
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    m_count, n_q, d = q64.shape
    if n_q % n_kv_heads:
        raise ValueError("query heads must be a multiple of the K/V heads")
    group = n_q // n_kv_heads
    k = dequantize_cache(k_codes, k_scales, n_kv_heads)
    v = dequantize_cache(v_codes, v_scales, n_kv_heads)
    t = k.shape[0]
    if k.shape[2] != d or v.shape != k.shape:
        raise ValueError("cache shapes do not match the queries")
    if t < m_count:
        raise ValueError("the cache must hold the M query tokens")
    out = np.zeros((m_count, n_q, d))
    for m in range(m_count):
        n_vis = visible_length(t, m_count, m)
        for h in range(n_q):
            g = h // group
            s = k[:n_vis, g, :] @ q64[m, h] / np.sqrt(d)
            p = np.exp(s - np.max(s))
            p /= np.sum(p)
            out[m, h] = p @ v[:n_vis, g, :]
    return out
