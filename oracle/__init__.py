"""CPU oracle for the W4A16 mixture-of-experts decode layer and the dense W4A16 GEMV.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 statement of what
the GPU library computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python
binding) never imports, calls or links anything here, and nothing here imports the
product package.  The two sides share no code: the oracle re-derives every format
rule from the source pages and from the OCP Microscaling FP4 (E2M1) definition.

Sources (cited by page title and section throughout):
  * "Lynn Engine" article (zingnex.cn), section "Native NVFP4 quantization support"
    and "Kernel optimisation history", stage P1: packed E2M1 codes with an FP16
    scale per 16 K-elements, read directly by a W4A16 matvec.
  * lynn-engine README (GitHub), status notes P28/P29 (gate/up + SiLU and the
    down weighted-sum contracts), P35/P20 (sorted top-k, order-free combine),
    P45 (one-call active-MoE ABI), P23 (int32 expert ids).
  * lynn-engine tutorials index, note 06 ("MoE router: softmax before or after
    top-K") and the Qwen 3.6 35B-A3B configuration block.
  * "cuda_inf" article (pure-CUDA engine on RTX 3060), section "2. INT4 weight
    quantization": symmetric int4 with one scale per group of 128.

Parity status of each function is stated in its module header.
"""

from .formats import (  # noqa: F401
    E2M1_GROUP,
    INT4_GROUP,
    FMT_E2M1,
    FMT_INT4,
    FMT_NVFP4,
    FMT_BF16,
    FMT_MXFP4,
    MX_BLOCK,
    E4M3_MAX,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    e2m1_value,
    int4_value,
    e4m3_value,
    f32_to_ue4m3,
    quantize_e2m1,
    quantize_int4,
    quantize_nvfp4,
    quantize_mxfp4,
    e8m0_value,
    mx_e4m3,
    quantize,
    pack_nibbles,
    unpack_nibbles,
    dequant,
    codes_bytes,
    scales_bytes,
)
from .ops import (  # noqa: F401
    gemv,
    router_probs,
    route,
    route_topk_softmax,
    shared_gate,
    expert_ffn,
    MoELayer,
    moe_experts,
    moe_forward,
    rel_l1,
    error_report,
)
