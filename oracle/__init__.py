"""Plain fp64 CPU oracle for absorbed MLA decode over a paged latent cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its Python binding) never
imports it, and it imports nothing from the product.

Everything is float64 numpy, written from the definitions on the pages:
  * the naive ("path A") and absorbed ("path B") score formulas of the MLA
    operator-teardown page (jh158.com), section 4;
  * the per-token latent row of 512 c_KV + 64 k_R values and the 64-token
    page of the same page, sections 1 and 3;
  * the split scan plus log-sum-exp reduction structure of the MI355X Kimi K3
    time-share study (jinnpan.com), "Inside the blocks" (stage 1 KV scan,
    stage 2 KV-split reduction);
  * the cache append with the decoupled RoPE key rotated in fp32 (teardown
    page, sections 3 and 4), with the frequency and pair layout readings
    stated beside the code;
  * the decompressed branch for chunks above the absorption threshold
    (teardown page, section 3 threshold, section 4 path A in two stages);
  * an 8-bit latent cache (FP8 E4M3 codes with one power-of-two scale per
    token, k_R kept in bf16), the analog of the teardown page's quantized
    latent gather (section 5), with the format readings stated beside it;
  * a 4-bit latent cache (OCP MXFP4: E2M1 codes with one E8M0 scale per 32
    latent dims, k_R kept in bf16), the same analog in the microscaling form
    the MI355X matrix cores read.

Each function is pinned by tests under ``tests/test_oracle*.py`` against
closed forms, brute-force loops, the pages' storage arithmetic and the
naive/absorbed identity. The pages' printed bf16 error magnitudes for their
absorption script are not reproducible and are not used as a pin.
"""
from .mla_oracle import (  # noqa: F401
    as_f64, bf16_bits, bf16_bits_to_f64, default_scale, gather_rows, absorb, visible_len,
    scores_absorbed, softmax_rows, attend_absorbed, decode_absorbed,
    decode_naive, up_proj, decode_split, combine, decode_rows,
    latent_row_elems, latent_row_bytes, mha_kv_bytes_per_token_layer,
    ROPE_BASE, rope_angles, rope_rotate, chunk_positions, append_latent,
    PREFILL_ABSORPTION_THRESHOLD, uses_absorption, decompress_kv, rope_keys, attend_mha,
    FP8_MAX, e4m3_value, e4m3_encode, fp8_scale_exponent, quantize_latent_fp8, dequantize_latent_fp8,
    fp8_page_bytes, pack_fp8_cache, unpack_fp8_pages, dequantize_fp8_pages, PagedQuantCache, PagedFp8Cache,
    E2M1_MAX, MX_BLOCK, e2m1_value, e2m1_encode, mx_scale_exponent, quantize_latent_mxfp4,
    dequantize_latent_mxfp4, mxfp4_page_bytes, pack_mxfp4_cache, unpack_mxfp4_pages, dequantize_mxfp4_pages,
    PagedMxfp4Cache,
)
