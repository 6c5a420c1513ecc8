// Instances of the MFMA attention kernel for bf16 inputs, head dimension 64.
#include "fa_fwd_mfma.h"

FA_MFMA_TABLE(mfma_variants_bf16_d64, __bf16, "bf16", FA_BF16, 64)
