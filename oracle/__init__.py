"""Plain CPU oracle of the TurboQuant KV-cache hot path (test infrastructure only).

This package is the slow, obviously correct reference that the HIP path is checked
against.  It is written from the pages, not from the HIP code, and shares no code
with it: nothing under ``kv_cache_vector_tq_amd/`` is imported here, and the product
never imports this package (only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it).

All floating point is fp64 unless a step fixes another precision (the stored
fp32 codebook tables, the bf16 rotation / sketch matrices).

Sources (page title, section):
  * "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru overview),
    paragraphs on the random rotation, the Lloyd-Max quantizer, the QJL residual
    correction and the data-oblivious property.
  * "Google TurboQuant простыми словами" (tproger.ru), section "Как работает TurboQuant",
    step 2 (QJL: Johnson-Lindenstrauss, zero bias, one extra bit), and section
    "Бенчмарки TurboQuant", list "Из независимых реализаций" (MSE 0.034 / 0.009,
    52 bytes per 128 values).

Modules and what pins each (tests/test_oracle_*.py):
  lloyd_max   Gaussian Lloyd-Max codebooks      pinned: closed form at 1 bit, quadrature,
                                                 printed MSE values, distortion-rate bounds
  params      SplitMix64, Box-Muller, Haar QR,  pinned: published SplitMix64 output,
              bf16 rounding                      QR uniqueness, orthogonality, bf16 bit cases
  quantize    rotate / scalar code / QJL sign   pinned: nearest-centroid brute force,
                                                 empirical MSE vs the printed figures,
                                                 QJL unbiasedness and variance closed form
  layout      packed cache layout (this repo's)  pinned: hand-written golden bytes,
                                                 round trip, 52-byte block accounting
  attention   decode attention from codes        pinned: dense dequantized softmax
                                                 attention, special cases (T=1, q=0)
"""
