// Internal interface between the C API (fa_api.cpp), the argument checks
// (fa_validate.cpp) and the kernels (fa_fwd_kernels.hip).  Not installed.
#ifndef FA_INTERNAL_H
#define FA_INTERNAL_H

#include <cstdint>

#include "fa.h"

// Functions also compiled for the device where hipcc builds them (plain C++
// elsewhere, e.g. the host-only sanitizer build of the argument checks).
#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// Entry i (0 .. B) of a packed offset array is valid if cu[0] = 0 and
// 0 <= cu[i] - cu[i-1] <= n_max (offsets non-decreasing, no sequence longer
// than the bound that sized the launch).  prev = cu[i-1] (unused for i = 0).
FA_HD inline bool seqlens_entry_ok(int i, int prev, int cur, int n_max) {
  if (i == 0) return cur == 0;
  const long long len = (long long)cur - (long long)prev;
  return len >= 0 && len <= (long long)n_max;
}

// The whole array (host memory): FA_OK or FA_ERR_SEQLENS.
inline int check_seqlens(const int* cu, int B, int n_max) {
  if (!cu) return FA_ERR_NULL;
  for (int i = 0; i <= B; ++i)
    if (!seqlens_entry_ok(i, i > 0 ? cu[i - 1] : 0, cu[i], n_max)) return FA_ERR_SEQLENS;
  return FA_OK;
}

// Query rows each wave owns (multiples of 32; with 64 the two 32-row blocks
// share every K/V operand read from LDS).
constexpr int rows_per_wave(int in_dtype) { return in_dtype == FA_F32 ? 32 : 32; }

// Waves per workgroup of the forward attention kernels.  16-bit inputs: 8
// (all eight share each K/V tile in LDS), except 4 at d = 64 under the
// causal mask.  There a workgroup's K/V walk is short next to its fixed
// costs (Q load, prologue, epilogue) and row blocks differ in length:
// smaller workgroups, more of them per CU, overlap one's prologue with
// another's main loop and even out the launch's end.  Without the mask,
// 8 waves' sharing of each tile is worth more.  fp32 inputs: 4.
constexpr int waves_per_wg(int in_dtype, int d, bool causal) {
  return in_dtype == FA_F32 || (d == 64 && causal) ? 4 : 8;
}

// Block-sparse attention: query rows and keys per block of a block mask,
// and the most 64-key tiles one sequence may have (the attention kernel
// keeps a list of them in LDS).
constexpr int kSparseBlock = 64;
constexpr int kMaxSparseTiles = 4096;

// How the launch covers the work.  A workgroup is waves_per_wg() waves; each
// wave owns rows_per_wave() query rows of one query head.  `hp` query heads that share
// one K/V head are packed into a workgroup (GQA), so one K/V tile in LDS
// serves them all; the workgroup then covers waves_per_wg * rows_per_wave / hp
// rows of each of those heads.
struct Plan {
  int hp;            // query heads per workgroup (1, 2 or 4)
  int rows_per_wg;   // query rows per head per workgroup
  int n_rblocks;     // row blocks per (sequence, head group): ceil(N / rows_per_wg)
  int n_hgroups;     // head groups: Hq / hp
  uint64_t total_wg; // B * n_hgroups * n_rblocks
};

// nw: waves per workgroup of the kernel the plan is for.
inline Plan make_plan_nw(int B, int Hq, int Hkv, int N, int in_dtype, int nw) {
  Plan p;
  const int G = Hq / Hkv;
  if (in_dtype == FA_F32) p.hp = 1;
  else p.hp = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  p.rows_per_wg = nw * rows_per_wave(in_dtype) / p.hp;
  p.n_rblocks = (int)(((long long)N + p.rows_per_wg - 1) / p.rows_per_wg);
  p.n_hgroups = Hq / p.hp;
  p.total_wg = (uint64_t)B * (uint64_t)p.n_hgroups * (uint64_t)p.n_rblocks;
  return p;
}

// The forward attention kernels' plan.
inline Plan make_plan(int B, int Hq, int Hkv, int N, int d, int in_dtype, bool causal) {
  return make_plan_nw(B, Hq, Hkv, N, in_dtype, waves_per_wg(in_dtype, d, causal));
}

// 64-key V^T tiles per (sequence, K/V head) in the packed-V workspace.
inline int vt_tiles(int N) { return (int)(((long long)N + 63) / 64); }

// Longest sequence (query or key count) the kernels take: their int index
// arithmetic (a row or key plus a tile or block size) stays far from
// overflow below it.
constexpr int kMaxSeqLen = 1 << 30;

// Bytes of the packed V^T workspace: B * Hkv * vt_tiles(N) tiles of d rows x
// 64 keys in 16 bits.  fp32 inputs need none.  Saturates at UINT64_MAX.
inline uint64_t workspace_bytes(int B, int Hkv, int N, int d, int in_dtype) {
  if (in_dtype == FA_F32 || B < 1 || Hkv < 1 || N < 1 || d < 1) return 0;
  const uint64_t tiles = (uint64_t)B * (uint64_t)Hkv * (uint64_t)vt_tiles(N);
  const uint64_t per = 128ull * (uint64_t)d;
  return tiles > UINT64_MAX / per ? UINT64_MAX : tiles * per;
}

inline uint64_t grid_size(int B, int Hq, int Hkv, int N, int d, int in_dtype) {
  // The larger of the two forward grids (with and without the mask);
  // UINT64_MAX (never a valid grid) for sizes the plan is not defined for.
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return UINT64_MAX;
  return make_plan(B, Hq, Hkv, N, d, in_dtype, true).total_wg;
}

// Checks of the attention arguments (Nq queries, Nk keys per sequence; the
// fa_fwd form has Nq = Nk and one offset array).  v_bytes is the extent of
// v used for the overlap test with o (0: the size of V itself).  Any finite
// scale is accepted.
int check_args(const void* q, const void* k, const void* v, const void* o,
               const float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
               int in_dtype, int out_dtype, uint64_t v_bytes = 0);

// Checks of the packed-V attention arguments (vt from fa_pack_v).
int check_packed_args(const void* q, const void* k, const void* vt, uint64_t vt_bytes,
                      const void* o, const float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                      int d, int causal, float scale, const int* cu_seqlens_q,
                      const int* cu_seqlens_k, int in_dtype, int out_dtype);
int check_pack_args(const void* v, const void* vt, uint64_t vt_bytes, int B, int Hkv, int N,
                    int d, const int* cu_seqlens, int in_dtype);

// Checks of the split-KV arguments (after check_packed_args): num_splits in
// [1, 256], the partial buffer (when num_splits > 1) present, 16-byte
// aligned, large enough and clear of o and lse, and the grid in range.
// Block mask arguments of fa_fwd_sparse*: pointer, broadcast counts, the
// key-tile limit, 16-bit inputs, and no overlap with o or lse.
int check_sparse_args(const void* block_mask, int mask_batches, int mask_heads, const void* o,
                      const float* lse, int B, int Hq, int Nq, int Nk, int d, int in_dtype,
                      int out_dtype, bool varlen);
uint64_t sparse_mask_bytes(int mask_batches, int mask_heads, int Nq, int Nk);

int check_split_args(const void* part, uint64_t part_bytes, const void* o, const float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits,
                     int in_dtype, int out_dtype, bool varlen);

struct LaunchArgs {
  const void* q; const void* k; const void* v; void* o; float* lse;
  const void* vt;      // packed V^T (16-bit inputs; v is then unused)
  const int* cu_seqlens;    // query offsets (varlen), or nullptr
  const int* cu_seqlens_k;  // key/value offsets (varlen), or nullptr
  int B, Hq, Hkv, N, Nk, d, causal;   // N: max query count, Nk: max key count
  float scale;
  int in_dtype, out_dtype;
  // Split-KV (16-bit inputs): n_splits > 1 writes partial results to o_part /
  // lse_part (split_workspace_bytes) and merges them into o / lse.
  int n_splits = 0;
  float* o_part = nullptr;
  float* lse_part = nullptr;
  // Block-sparse (16-bit inputs): uint8 mask [mask_batches][mask_heads]
  // [ceil(N/64)][ceil(Nk/64)], or nullptr.
  const uint8_t* block_mask = nullptr;
  int mask_batches = 0, mask_heads = 0;
};

// Bytes of the split-KV partials: n_splits x B x Hq x Nq rows of d fp32
// values plus one fp32 L each.  Saturates at UINT64_MAX.
inline uint64_t split_workspace_bytes(int B, int Hq, int Nq, int d, int n_splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || d < 1 || n_splits < 1) return 0;
  const uint64_t rows = (uint64_t)n_splits * (uint64_t)B * (uint64_t)Hq * (uint64_t)Nq;
  const uint64_t per = 4ull * ((uint64_t)d + 1);
  return rows > UINT64_MAX / per ? UINT64_MAX : rows * per;
}

// Shapes that run the decode kernel: 16-bit inputs, dense, and the G query
// heads of a K/V head times the query rows per sequence fit one 32-row
// MFMA block.
inline bool use_decode(int in_dtype, int Hq, int Hkv, int Nq, bool sparse) {
  return in_dtype != FA_F32 && !sparse && Hkv > 0 && Nq >= 1 &&
         (long long)(Hq / Hkv) * Nq <= 32;
}

// A split count that fills the GPU when the grid alone would not: used for
// decode-like shapes (few query rows per sequence).  1 = no split.
int suggest_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int in_dtype, int cus);

// Enqueue the kernel for already-checked arguments.  Returns FA_OK or
// FA_ERR_LAUNCH.  `stream` is a hipStream_t.
int launch_fwd(const LaunchArgs& a, void* stream);

// Enqueue the V^T packing kernel (16-bit inputs) for checked arguments.
int launch_vt_pack(const void* v, void* vt, int B, int Hkv, int N, int d, const int* cu_seqlens,
                   int in_dtype, void* stream);

// Backward pass (16-bit inputs).
struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;
  void* dq; void* dk; void* dv;
  const int* cu_seqlens;
  int B, Hq, Hkv, N, d, causal;
  float scale;
  int in_dtype, o_dtype, grad_dtype;
  void* workspace;
};
// Bytes of the backward's workspace: the rows' D and L * log2(e), fp32
// [B][Hq][N] each, each padded to 256 bytes (as laid out by the backward's
// launch).  Saturates at UINT64_MAX; 0 for non-positive sizes.
inline uint64_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  (void)Hkv;
  (void)d;
  if (B < 1 || Hq < 1 || N < 1) return 0;
  const uint64_t rows = (uint64_t)B * (uint64_t)Hq * (uint64_t)N;   // < 2^93: checked below
  if ((uint64_t)B * (uint64_t)Hq > UINT64_MAX / (uint64_t)N || rows > (UINT64_MAX - 512) / 8)
    return UINT64_MAX;
  return 2 * ((rows * 4 + 255) & ~255ull);
}
int check_bwd_args(const BwdArgs& a, uint64_t ws_bytes);
int launch_bwd(const BwdArgs& a, void* stream);

// Static name of the kernel instance for these settings, or nullptr.
const char* kernel_name(int in_dtype, int d, int causal, int varlen, int out_dtype);
// The same for fa_fwd_kv with Hq, Hkv and the query count Nq (the decode
// kernel where use_decode holds), block-sparse or not, and with V packed
// (vpack) or row-major.
const char* kernel_name_kv(int in_dtype, int d, int causal, int varlen, int out_dtype, int Hq,
                           int Hkv, int Nq, int sparse = 0, int vpack = 0);

// Size of the library's fixed device scratch (fa_fwd_kv_split_noalloc's
// split-KV partials), and its device address on the current device
// (nullptr if unavailable).  Calls that overlap on one device share it.
constexpr uint64_t kNoAllocScratchBytes = 16ull << 20;
void* noalloc_scratch();

// The launch order fa_debug_force_order (or FA_FORCE_ORDER) sets: -1 for the
// library's own choice, else bit 0 = XCD remap, bit 1 = row-block-major.
int forced_order();

// Debug mode (FA_DEBUG=1): check a packed offset array (B + 1 entries in
// device memory) on `stream` and wait for the outcome: FA_OK,
// FA_ERR_SEQLENS if an entry fails seqlens_entry_ok, or FA_ERR_LAUNCH.
// Synchronises `stream`; calls are serialised.
int debug_check_seqlens(const int* cu, int B, int n_max, void* stream);

}  // namespace fa

#endif  // FA_INTERNAL_H
