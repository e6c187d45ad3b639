"""Oracle byte accounting of the numeric KV payload.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "KV quantization axes ...", section "Scales occupy bytes too": the
payload counts the integer codes and the float32 scales and nothing else
(no object headers, allocators or workspaces); for int8 codes with keys per
channel and values per token the total is 2ND + 4D + 4N bytes.

The functions below count bytes from the shapes of the arrays the oracle
actually produces, so the printed table pins both the formula and the
grouping shapes.
"""

from . import codec


def int8_payload_bytes(k_codes, k_scales, v_codes, v_scales):
    """Bytes of int8 codes (one byte each) plus float32 scales."""
    return (k_codes.size + v_codes.size) + 4 * (k_scales.size + v_scales.size)


def float32_payload_bytes(n, d):
    """Unquantized float32 K and V."""
    return 2 * n * d * 4


def cache_stream_bytes(n_sink, n_quant, n_tail, d, k_bits, v_bits, G, Gv,
                       mixed=False, n_bf16=0, n_int4=0):
    """Bytes a decode step must read for one (batch, KV head) stream.

    Packed code rows (whole uint32 words per token), float32 scales, and
    fp16 K and V rows for the sink and the tail.  For mixed keys each group
    also stores one class byte per channel.
    """
    n_groups = n_quant // G
    b = 0
    if mixed:
        n2 = d - n_bf16 - n_int4
        b += n_quant * (2 * n_bf16 + 4 * codec.words_per_row(n_int4, 4)
                        + 4 * codec.words_per_row(n2, 2))
        b += n_groups * (4 * (n_int4 + n2) + d)
    else:
        b += n_quant * 4 * codec.words_per_row(d, k_bits)
        b += n_groups * d * 4
    b += n_quant * 4 * codec.words_per_row(d, v_bits)
    b += n_quant * (d // Gv) * 4
    b += (n_sink + n_tail) * d * 2 * 2
    return b
