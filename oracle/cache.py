"""Oracle of the quantized KV cache: sink, quantized groups, residual tail.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources (page title, section):

* "MixKVQ ...", Figure 4 caption: keys are quantized per channel and values
  per token, with a full-precision buffer of R recent tokens in front of the
  quantized cache; key salience is refreshed every R tokens.
* "KVQuant ...", summary and "Measured effects" table: the first token (the
  attention sink) stays in fp16; keys per channel, values per token; the
  residual-buffer baseline they compare against keeps 128 recent tokens.
* "KV quantization axes ...", "What rows and columns mean": the symmetric
  rule used for every quantized group (oracle.codec).

Readings where the pages leave a step open:

* flush-on-overflow: the tail holds up to R tokens; when one more token
  arrives at a full tail, its oldest G tokens are quantized together as one
  key group (and per token for values), R being a multiple of G;
* sink and tail keep both K and V verbatim in fp16;
* uniform caches quantize keys at k_bits and values at v_bits; mixed caches
  rank each flushed key group's channels by salience (oracle.salience) and
  store n_bf16 channels as bf16, n_int4 as int4 and the rest as int2, each
  class in ascending channel order.
"""

from dataclasses import dataclass

import numpy as np

from . import codec, salience


@dataclass
class CacheConfig:
    B: int
    Hkv: int
    D: int
    S: int          # sink tokens kept in fp16
    R: int          # residual tail capacity (multiple of G)
    G: int          # key group, tokens
    Gv: int         # value group, channels
    k_bits: int
    v_bits: int
    mixed: bool = False
    n_bf16: int = 0
    n_int4: int = 0

    def check(self):
        if self.G <= 0 or self.R < self.G or self.R % self.G:
            raise ValueError("R must be a positive multiple of G")
        if self.D % self.Gv:
            raise ValueError("Gv must divide D")
        codec.qmax_for_bits(self.k_bits)
        codec.qmax_for_bits(self.v_bits)
        if self.mixed and self.n_bf16 + self.n_int4 > self.D:
            raise ValueError("class counts exceed D")


def tail_length(n_past_sink, R, G):
    """Closed form of the tail length after n tokens past the sink."""
    if n_past_sink <= R:
        return n_past_sink
    return R - G + ((n_past_sink - R - 1) % G) + 1


class _Stream:
    def __init__(self, d):
        z16 = np.zeros((0, d), np.float16)
        self.sink_k, self.sink_v = z16, z16.copy()
        self.tail_k, self.tail_v = z16.copy(), z16.copy()
        self.groups = []     # one dict per flushed key group
        self.v_codes, self.v_scales = [], []   # one array per flushed group


class Cache:
    def __init__(self, cfg: CacheConfig):
        cfg.check()
        self.cfg = cfg
        self.streams = [[_Stream(cfg.D) for _ in range(cfg.Hkv)]
                        for _ in range(cfg.B)]
        self.I = np.ones((cfg.B, cfg.Hkv, cfg.D), np.float64)
        self.n_tokens = 0

    # -- salience -----------------------------------------------------------
    def salience_select(self, q_win):
        """q_win: [B][W][Hq][D] float16; sets I for all later flushes."""
        q = np.asarray(q_win)
        for b in range(self.cfg.B):
            self.I[b] = salience.intensity(q[b], self.cfg.Hkv)

    # -- append ---------------------------------------------------------------
    def append(self, k_new, v_new):
        """k_new, v_new: [B][Hkv][n][D] float16, appended in token order.

        Tokens fill the sink first; the rest join the tail, and whenever the
        tail holds more than R tokens its oldest G are flushed.  Flushing
        after the whole batch joined gives the same groups as flushing
        before each token that would overflow a full tail (the groups are
        always the oldest G tail tokens, in order); the tests check this
        against one-token-at-a-time appends.
        """
        k = np.asarray(k_new)
        v = np.asarray(v_new)
        if k.dtype != np.float16 or v.dtype != np.float16:
            raise TypeError("append takes float16 K and V")
        cfg = self.cfg
        if not (np.all(np.isfinite(k)) and np.all(np.isfinite(v))):
            raise codec.NonFiniteInput("NaN/Inf input is rejected")
        n = k.shape[2]
        for b in range(cfg.B):
            for h in range(cfg.Hkv):
                st = self.streams[b][h]
                take = min(cfg.S - st.sink_k.shape[0], n)
                st.sink_k = np.concatenate([st.sink_k, k[b, h, :take]])
                st.sink_v = np.concatenate([st.sink_v, v[b, h, :take]])
                st.tail_k = np.concatenate([st.tail_k, k[b, h, take:]])
                st.tail_v = np.concatenate([st.tail_v, v[b, h, take:]])
                while st.tail_k.shape[0] > cfg.R:
                    self._flush(b, h, st)
        self.n_tokens += n

    def _flush(self, b, h, st):
        cfg = self.cfg
        kg = st.tail_k[:cfg.G]
        vg = st.tail_v[:cfg.G]
        st.tail_k = st.tail_k[cfg.G:]
        st.tail_v = st.tail_v[cfg.G:]
        if cfg.mixed:
            st.groups.append(self._mixed_group(b, h, kg))
        else:
            codes, scales = codec.quantize_k(kg, cfg.k_bits, cfg.G)
            st.groups.append({"codes": codes.astype(np.int8),
                              "scales": scales[0]})
        vc, vs = codec.quantize_v(vg, cfg.v_bits, cfg.Gv)
        st.v_codes.append(vc.astype(np.int8))
        st.v_scales.append(vs)

    def _mixed_group(self, b, h, kg):
        cfg = self.cfg
        S = salience.group_key_scale(kg)
        cls = salience.classes(self.I[b, h], S, cfg.n_bf16, cfg.n_int4)
        grp = {"cls": cls}
        ch_bf = [c for c in range(cfg.D) if cls[c] == salience.CLASS_BF16]
        ch_i4 = [c for c in range(cfg.D) if cls[c] == salience.CLASS_INT4]
        ch_i2 = [c for c in range(cfg.D) if cls[c] == salience.CLASS_INT2]
        grp["ch_bf16"], grp["ch_int4"], grp["ch_int2"] = ch_bf, ch_i4, ch_i2
        kf = kg.astype(np.float32)
        grp["bf16"] = codec.f32_to_bf16_bits(kf[:, ch_bf]) if ch_bf else \
            np.zeros((cfg.G, 0), np.uint16)
        for name, chans, bits in (("int4", ch_i4, 4), ("int2", ch_i2, 2)):
            if chans:
                codes, scales = codec.quantize_k(kg[:, chans], bits, cfg.G)
                scales = scales[0]
            else:
                codes = np.zeros((cfg.G, 0), np.int32)
                scales = np.zeros(0, np.float32)
            grp[name + "_codes"] = codes.astype(np.int8)
            grp[name + "_scales"] = scales
        return grp

    # -- views ------------------------------------------------------------------
    def counts(self):
        st = self.streams[0][0]
        return (st.sink_k.shape[0], len(st.groups) * self.cfg.G,
                st.tail_k.shape[0])

    def dequantized(self, b, h):
        """(K_hat, V_hat) float64 [N][D] in token order: sink, groups, tail."""
        cfg = self.cfg
        st = self.streams[b][h]
        ks, vs = [], []
        if st.sink_k.shape[0]:
            ks.append(st.sink_k.astype(np.float64))
            vs.append(st.sink_v.astype(np.float64))
        for grp in st.groups:
            ks.append(self._dequant_group(grp))
        if st.groups:
            vc = np.concatenate(st.v_codes)
            vsc = np.concatenate(st.v_scales)
            vs.append(codec.dequant(vc, codec.expand_v_scales(vsc, cfg.D,
                                                              cfg.Gv)))
        if st.tail_k.shape[0]:
            ks.append(st.tail_k.astype(np.float64))
            vs.append(st.tail_v.astype(np.float64))
        if not ks:
            z = np.zeros((0, cfg.D), np.float64)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def _dequant_group(self, grp):
        cfg = self.cfg
        if not cfg.mixed:
            return codec.dequant(grp["codes"],
                                 np.broadcast_to(grp["scales"],
                                                 grp["codes"].shape))
        out = np.zeros((cfg.G, cfg.D), np.float64)
        if grp["ch_bf16"]:
            out[:, grp["ch_bf16"]] = codec.bf16_bits_to_f32(
                grp["bf16"]).astype(np.float64)
        for name in ("int4", "int2"):
            chans = grp["ch_" + name]
            if chans:
                out[:, chans] = codec.dequant(
                    grp[name + "_codes"],
                    np.broadcast_to(grp[name + "_scales"],
                                    grp[name + "_codes"].shape))
        return out

    def export(self):
        """Canonical arrays, the layout the library's export produces."""
        cfg = self.cfg
        B, H, D = cfg.B, cfg.Hkv, cfg.D
        ns, nq, nt = self.counts()
        ng = nq // cfg.G
        out = {
            "sink_k": np.zeros((B, H, ns, D), np.float16),
            "sink_v": np.zeros((B, H, ns, D), np.float16),
            "tail_k": np.zeros((B, H, nt, D), np.float16),
            "tail_v": np.zeros((B, H, nt, D), np.float16),
            "v_codes": np.zeros((B, H, nq, codec.words_per_row(D, cfg.v_bits)),
                                np.uint32),
            "v_scales": np.zeros((B, H, nq, D // cfg.Gv), np.float32),
        }
        if cfg.mixed:
            n2 = D - cfg.n_bf16 - cfg.n_int4
            out["k_class"] = np.zeros((B, H, ng, D), np.uint8)
            out["k_bf16"] = np.zeros((B, H, nq, cfg.n_bf16), np.uint16)
            out["k_int4"] = np.zeros(
                (B, H, nq, codec.words_per_row(cfg.n_int4, 4)), np.uint32)
            out["k_int2"] = np.zeros(
                (B, H, nq, codec.words_per_row(n2, 2)), np.uint32)
            out["k_scales"] = np.zeros((B, H, ng, cfg.n_int4 + n2),
                                       np.float32)
        else:
            out["k_codes"] = np.zeros(
                (B, H, nq, codec.words_per_row(D, cfg.k_bits)), np.uint32)
            out["k_scales"] = np.zeros((B, H, ng, D), np.float32)
        for b in range(B):
            for h in range(H):
                st = self.streams[b][h]
                out["sink_k"][b, h] = st.sink_k
                out["sink_v"][b, h] = st.sink_v
                out["tail_k"][b, h] = st.tail_k
                out["tail_v"][b, h] = st.tail_v
                if nq:
                    out["v_codes"][b, h] = codec.pack_rows(
                        np.concatenate(st.v_codes), cfg.v_bits)
                    out["v_scales"][b, h] = np.concatenate(st.v_scales)
                for gi, grp in enumerate(st.groups):
                    t0 = gi * cfg.G
                    sl = slice(t0, t0 + cfg.G)
                    if cfg.mixed:
                        out["k_class"][b, h, gi] = grp["cls"]
                        if cfg.n_bf16:
                            out["k_bf16"][b, h, sl] = grp["bf16"]
                        if cfg.n_int4:
                            out["k_int4"][b, h, sl] = codec.pack_rows(
                                grp["int4_codes"], 4)
                        if grp["int2_codes"].shape[1]:
                            out["k_int2"][b, h, sl] = codec.pack_rows(
                                grp["int2_codes"], 2)
                        out["k_scales"][b, h, gi] = np.concatenate(
                            [grp["int4_scales"], grp["int2_scales"]])
                    else:
                        out["k_codes"][b, h, sl] = codec.pack_rows(
                            grp["codes"], cfg.k_bits)
                        out["k_scales"][b, h, gi] = grp["scales"]
        return out
