// Instances of the MFMA attention kernel for bf16 inputs, head dimension 128.
#include "fa_fwd_mfma.h"

FA_MFMA_TABLE(mfma_variants_bf16_d128, __bf16, "bf16", FA_BF16, 128)
