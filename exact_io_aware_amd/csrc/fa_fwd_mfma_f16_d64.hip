// Instances of the MFMA attention kernel for f16 inputs, head dimension 64.
#include "fa_fwd_mfma.h"

FA_MFMA_TABLE(mfma_variants_f16_d64, _Float16, "f16", FA_F16, 64)
