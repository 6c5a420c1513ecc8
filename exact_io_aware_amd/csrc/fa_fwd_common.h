// Launch parameters and the instance tables shared by the forward kernels'
// translation units (the MFMA attention kernel is instantiated in one unit
// per input type and head dimension, so they compile in parallel).
#ifndef FA_FWD_COMMON_H
#define FA_FWD_COMMON_H

#include <cstdint>

#include "fa.h"
#include "fa_internal.h"

namespace fa {

struct FwdParams {
  const void* q; const void* k; const void* v; void* o; float* lse;
  const int* cu_seqlens;   // query offsets (varlen)
  const int* cu_seqlens_k; // key/value offsets (varlen)
  int N, Nk, Hq, G;        // max query count, max key count, query heads, Hq / Hkv
  int hp, rows_per_wg, n_rblocks, n_hgroups, total_wg, xcd_remap;
  // rb_major (causal): row-block slot s of every unit is launched before slot
  // s + 1 of any, slot s being a sequence's s-th longest row block.
  int rb_major, n_units;
  float scale_log2;        // |scale| * log2(e) (log2(e) when scale = 0)
  // How Q enters the scores: 0 as stored; 1 negated (scale < 0: the scores
  // scale * q.k equal |scale| * (-q).k, and negating a 16-bit or fp32 value
  // is exact); 2 zero (scale = 0: every visible score is 0).
  int q_mode;
  const void* vt;          // packed V^T tiles (16-bit inputs), see fa_vt_pack
  int Hkv, vt_ntiles;      // K/V heads; 64-key tiles per (sequence, K/V head)
  // Split-KV: n_splits > 1 cuts each unit's keys into ranges of split_tiles
  // 64-key tiles; workgroup (unit, split) writes the normalised partial O
  // (fp32, [split][B][Hq][N][d]) and partial L ([split][B][Hq][N]).
  int n_splits, split_tiles, B;
  float* o_part; float* lse_part;
  long long q_bs, q_hs, q_rs;    // element strides of q (and o): batch, head, row
  long long kv_bs, kv_hs, kv_rs; // element strides of k and v
  // Block-sparse: uint8 mask over 64 x 64 (query row, key) blocks; entry
  // (b, h, i, j) at mask_bs * b + mask_hs * h + mask_nkb * i + j (a stride
  // is 0 where one mask serves every sequence or head).
  const uint8_t* block_mask;
  long long mask_bs, mask_hs;
  int mask_nkb;
};

typedef void (*KernelFn)(FwdParams);

// One instance of the MFMA attention kernel.  vpack: V comes as packed V^T
// tiles (fa_pack_v) instead of the row-major V itself.
struct Variant {
  int in_dtype, d, causal, varlen, out_dtype, sparse, vpack;
  KernelFn fn;
  const char* name;
};

// The instances of each translation unit: pointer to the table, count in *n.
const Variant* mfma_variants_bf16_d64(int* n);
const Variant* mfma_variants_bf16_d128(int* n);
const Variant* mfma_variants_f16_d64(int* n);
const Variant* mfma_variants_f16_d128(int* n);

}  // namespace fa

#endif  // FA_FWD_COMMON_H
