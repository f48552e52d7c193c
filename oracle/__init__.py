"""CPU oracle for the fused attention forward pass and the paged split-KV decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
anything in this package: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

What it computes is the plain definition of softmax attention, in float64, with
the full score matrix materialised:

    O = softmax(Q K^T * scale [+ mask]) V,   scale = 1/sqrt(D)

("Agent 帮我写 CUDA：一个 Softmax Attention 算子的开发全记录", section 二
"实验环境", reference-baseline paragraph and the note on D; section 四, the
tiled-attention flow, whose online-softmax recurrence is an exact rewriting of
this definition). The mask variants (causal, sliding window, tanh softcap),
grouped-query heads, ragged batches, paged KV and split-KV decode are the
scenario axes named in "Ask, Don't Equip: Question-Driven Coding Agents for
Deep Kernel Optimization", section 研究动机; the pages name them without
defining them, and the readings taken here are:

* causal, aligned bottom-right: key j is allowed for query i iff
  j <= i + (Nk - Nq);
* sliding window W > 0: additionally j > i + (Nk - Nq) - W (the W most recent
  keys, the diagonal included);
* softcap c > 0: s <- c * tanh(s / c) applied to the scaled score, before the
  mask;
* grouped heads: query head h reads KV head floor(h / (Hq / Hkv));
* a fully masked row gives O = 0 and LSE = -inf;
* LSE is the natural-log log-sum-exp of the final (scaled, capped, masked)
  scores;
* attention sink ("attention-sink" in the same list): an optional logit sigma_h
  per query head that joins every row's normalisation as a score with no value
  (exp(sigma_h) is added to the denominator and to the LSE's sum); a row with no
  allowed key then gives O = 0 and LSE = sigma_h.

Function pins (see tests/test_oracle_*.py): brute-force scalar loops, the
page's online recurrence, closed forms (identical keys, dominant key, N = 1,
D = 1), invariants (shift, permutation, GQA = MHA, varlen = concatenation,
paged = dense, chunked paged prefill = brute force with
scalar page indexing and = decode at one query, page-permutation invariance,
split/combine associativity, the sink (brute force, one-key closed form, the
rescaling identity O_sink = O e^LSE / (e^LSE + e^sigma), a negligible sink), the fp8
prefill (brute force on codes decoded bit by bit, the scale laws), the backward (central
finite differences of sum(dO * O), float64 autograd through a separately written forward,
closed forms for one key and for identical keys), softcap and window limits) and
library special cases (torch's bf16 / fp16 / float8_e4m3fn conversions).
"""
from .numerics import (bf16_bits_to_f64, f16_bits_to_f64, e4m3_code_table, e4m3_codes_to_f64,
                       default_scale, tensor_to_f64)
from .attention import (sdpa_fp64, prefill_dense, prefill_varlen, prefill_fp8, gather_pages, decode_paged,
                        prefill_paged, combine_partials, attention_probs, sdpa_backward_fp64,
                        prefill_backward_dense)

__all__ = [
    "bf16_bits_to_f64", "f16_bits_to_f64", "e4m3_code_table", "e4m3_codes_to_f64",
    "default_scale", "tensor_to_f64", "sdpa_fp64", "prefill_dense", "prefill_varlen", "prefill_fp8",
    "gather_pages", "decode_paged", "prefill_paged", "combine_partials", "attention_probs",
    "sdpa_backward_fp64", "prefill_backward_dense",
]
