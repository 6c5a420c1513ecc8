/*
 * fa.h — C ABI of libfa, an exact IO-aware attention forward pass
 * ("FlashAttention") for AMD Instinct MI355X (gfx950).
 *
 * The operation (fa_fwd): for every sequence b and query head h,
 *
 *     O[b,h] = softmax(scale * Q[b,h] K[b,g]^T) V[b,g],   g = h / (Hq/Hkv)
 *     L[b,h,r] = ln sum_c exp(scale * Q[b,h,r] . K[b,g,c])   (visible c)
 *
 * - The formula is the standard attention formula of the Kotaemon page
 *   ("Kotaemon FlashAttention应用：加快注意力计算", formula paragraph).
 * - The method: Q is cut into row blocks; for each row block the K/V blocks
 *   are streamed through on-chip memory; each block's scores update a running
 *   row maximum and normaliser, so the result equals the formula exactly
 *   (Kotaemon page, method list and the exactness paragraph after it;
 *   HolySheep Flash Attention article, Chinese edition, section
 *   "IO 感知的算法设计").  The N x N score matrix is never written to memory.
 * - O and the per-row normaliser L are both returned, as in the tiling
 *   sketch of the HolySheep article, French edition (section "Principe
 *   fondamental : tiling et streaming"); L is read as the natural-log
 *   logsumexp of the scaled, masked scores.
 * - causal = 1 masks key c for query r when c > r (top-left alignment,
 *   indices within the sequence), consistent with the manual chunking recipe
 *   of the French HolySheep article ("Erreurs courantes", item 1).
 * - Grouped-query attention: Hq must be a multiple of Hkv; query head h reads
 *   K/V head h / (Hq/Hkv) (contiguous groups; the transformer memory page
 *   "Empreinte mémoire et calcul des couches Transformer dans les LLM en
 *   production" uses H_KV = 8 with d_head = 128).
 *
 * Layouts (all contiguous, head dimension fastest):
 * - fixed length (cu_seqlens == NULL):
 *       q, o   [B][Hq][N][d]       k, v   [B][Hkv][N][d]
 * - packed variable length (cu_seqlens != NULL): B sequences packed token
 *   by token; cu_seqlens is a DEVICE int32 array [B+1] with cu_seqlens[0] = 0
 *   and non-decreasing offsets; T = cu_seqlens[B]; N must be >= the longest
 *   sequence length (it sizes the launch, so no device value is read on the
 *   host):
 *       q, o   [T][Hq][d]          k, v   [T][Hkv][d]
 * - lse is float32 [B][Hq][N] in both cases.  In the packed case the rows
 *   r >= length of sequence b are left untouched.
 *
 * Types: q, k and v share in_dtype (FA_F32, FA_F16 or FA_BF16).  o is
 * written in out_dtype, which is FA_F32 or in_dtype.  Scores, softmax
 * statistics and accumulators are fp32; P is rounded to in_dtype (round to
 * nearest even) for the P.V contraction; the normaliser is summed from the
 * unrounded fp32 P (bf16) or from the rounded P the P.V contraction uses
 * (fp16).
 *
 * Supported: d in {64, 128}; B, Hq, Hkv, N >= 1; Hq % Hkv == 0; causal in
 * {0, 1}; any finite scale (scale < 0 is computed as |scale| with Q
 * negated, scale = 0 as Q = 0: both exact).  No dropout, no arbitrary mask.
 *
 * Ownership and threading: every pointer is a device pointer owned by the
 * caller.  fa_fwd (and fa_fwd_kv, fa_fwd_sparse) is one kernel launch that
 * reads q, k, v and writes o and lse: it allocates nothing, keeps no
 * workspace and no per-call state, never splits the keys over workgroups
 * and never synchronises (V is read transposed on chip, so no transposed
 * copy of it is made).  The work is enqueued on `stream` (a hipStream_t;
 * NULL is the default stream) and fa_fwd returns at once.  Calls are
 * thread-safe; calls on different streams may run concurrently.  o must not
 * overlap q, k, v or lse.
 *
 * Errors: arguments are checked before anything is enqueued; on failure
 * nothing is launched and a negative fa_status is returned.  Pointers q, k,
 * v, o must be 16-byte aligned, lse and cu_seqlens 4-byte aligned.  A device
 * that is not gfx950 gives FA_ERR_DEVICE; a launch failure gives
 * FA_ERR_LAUNCH.  Corrupt cu_seqlens contents (cu[0] != 0, decreasing
 * offsets, a length above N) are not detected in normal operation, where
 * checking them would need a device-to-host read: the caller must pass valid
 * offsets.  With the environment variable FA_DEBUG=1 (read once per
 * process) every entry point that takes packed offsets first checks them
 * on the device and waits for the outcome: corrupt offsets give
 * FA_ERR_SEQLENS and no attention kernel runs.  That mode synchronises the
 * stream (it cannot be captured into a graph) and serialises the checks of
 * concurrent calls.  The Kotaemon page's caveats warn that a misconfigured
 * fast path fails silently; this mode makes that failure loud.  Offsets
 * past the caller's buffers cannot be detected (their extent is not
 * passed).  Nothing is printed and no exception crosses the ABI.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,     /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,    /* B, Hq, Hkv or N < 1, causal not 0/1, or size overflow */
  FA_ERR_HEADDIM = -3,  /* d not in {64, 128} */
  FA_ERR_GQA = -4,      /* Hq not a multiple of Hkv */
  FA_ERR_DTYPE = -5,    /* unknown in_dtype, or out_dtype not in {FA_F32, in_dtype} */
  FA_ERR_ALIGN = -6,    /* pointer misaligned */
  FA_ERR_ALIAS = -7,    /* o overlaps q, k, v or lse */
  FA_ERR_SCALE = -8,    /* scale not finite (backward: or not > 0) */
  FA_ERR_DEVICE = -9,   /* current device is not gfx950, or no device */
  FA_ERR_LAUNCH = -10,  /* the kernel launch failed */
  FA_ERR_WORKSPACE = -11, /* a caller workspace below its stated size */
  FA_ERR_ALLOC = -12,   /* reserved: no entry point allocates memory */
  FA_ERR_SEQLENS = -13, /* FA_DEBUG=1 only: corrupt cu_seqlens contents */
  FA_ERR_SCRATCH = -14  /* fa_fwd_kv_split_noalloc: partials above the fixed scratch */
} fa_status;

/* Exact attention forward (see the header comment).  q, k, v: inputs in
 * in_dtype; o: output in out_dtype; lse: float32 logsumexp; stream: a
 * hipStream_t or NULL.  Returns FA_OK or a negative fa_status. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           const int* cu_seqlens, void* stream, int in_dtype, int out_dtype);

/* Bytes of the packed-V layout that fa_pack_v fills and the *_packed entry
 * points read, for 16-bit inputs: B * Hkv * ceil(N / 64) tiles of d * 64
 * values (d * 128 bytes each).  0 for fp32 inputs and for unsupported d or
 * dtype.
 *
 * Why (a gfx950 design choice, not from the pages): the P.V product of each
 * key block takes V^T as its matrix operand.  fa_fwd reads V's rows into
 * on-chip memory and transposes them there (two transposing reads per
 * operand).  A decode loop, which keeps its K/V cache from call to call, can
 * keep V in this packed form instead (the operand is then one 16-byte read)
 * and re-pack only the tile holding each new token. */
size_t fa_workspace_bytes(int B, int Hkv, int N, int d, int in_dtype);

/* Pack V (layout as for fa_fwd, in_dtype FA_F16 or FA_BF16) into vt: for
 * every sequence b, K/V head g and 64-key tile t, the tile transposed (d rows
 * of 64 keys, 128 bytes per row; keys past the sequence end zero) at byte
 * offset ((b * Hkv + g) * ceil(N/64) + t) * d * 128.  Within each group of
 * 16 keys of a row, position j holds key (j % 4) + 8 * ((j / 4) % 2) +
 * 4 * (j / 8) of the group (the order of the P.V operand's fragments).  Tiles wholly past a
 * sequence's end are not written.  vt (16-byte aligned, vt_bytes >=
 * fa_workspace_bytes) must not overlap v.  Enqueued on `stream`; returns
 * FA_OK or a negative fa_status (FA_ERR_DTYPE for fp32 inputs) before
 * anything is enqueued. */
int fa_pack_v(const void* v, void* vt, size_t vt_bytes, int B, int Hkv, int N, int d,
              const int* cu_seqlens, void* stream, int in_dtype);

/* fa_fwd for 16-bit inputs with V given as fa_pack_v's output vt (packed
 * with the same B, Hkv, N, d, cu_seqlens and in_dtype, and enqueued before
 * this call on the same stream, or otherwise complete).  Same results as
 * fa_fwd, bit for bit; allocates nothing.  Errors as fa_fwd, plus
 * FA_ERR_WORKSPACE, and FA_ERR_DTYPE for fp32 inputs. */
int fa_fwd_packed(const void* q, const void* k, const void* vt, size_t vt_bytes, void* o,
                  float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                  const int* cu_seqlens, void* stream, int in_dtype, int out_dtype);

/* Queries against a longer key/value sequence (chunked prefill).  As
 * fa_fwd, but each sequence has nq query rows and nk key/value rows, and the
 * queries are the LAST nq tokens of the sequence: with causal = 1, query
 * row r sees keys c <= r + nk - nq (bottom-right alignment).  This is the
 * manual chunking recipe of the French HolySheep article ("Erreurs
 * courantes", item 1): the query chunk [i, i+c) attends to the key prefix
 * [0, i+c).  nq = nk gives fa_fwd.  A row that sees no key (causal with
 * nq > nk, or nk = 0 in a packed batch) gets O = 0 and L = -inf.
 *
 * Layouts: fixed (both offset arrays NULL): q, o [B][Hq][Nq][d],
 * k, v [B][Hkv][Nk][d], lse [B][Hq][Nq].  Packed: cu_seqlens_q and
 * cu_seqlens_k are DEVICE int32 arrays [B+1] (both given, or neither),
 * q, o [Tq][Hq][d], k, v [Tk][Hkv][d]; Nq and Nk bound the longest query
 * and key counts; lse [B][Hq][Nq] with rows past a sequence's nq untouched.
 * Errors as fa_fwd (FA_ERR_NULL if only one offset array is given; Nq, Nk
 * must be >= 1). */
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream,
              int in_dtype, int out_dtype);

/* fa_fwd_kv for 16-bit inputs with V packed by fa_pack_v (called with N = Nk
 * and cu_seqlens = cu_seqlens_k).  Allocates nothing. */
int fa_fwd_kv_packed(const void* q, const void* k, const void* vt, size_t vt_bytes, void* o,
                     float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                     float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
                     void* stream, int in_dtype, int out_dtype);

/* Split-KV (decode).  With few query rows per sequence (decode: one new
 * token per sequence against its KV cache) the grid has too few workgroups
 * to keep the GPU's memory system busy, so each unit's keys are cut into
 * num_splits ranges processed by separate workgroups.  Each writes its
 * range's normalised partial output and logsumexp into `part`; a merge pass
 * then forms L = ln sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s, the
 * same normaliser algebra as the online softmax (Kotaemon page, method list)
 * applied across ranges, so the result is the exact attention of
 * fa_fwd_kv.
 *
 * fa_num_splits: a split count for these sizes on the current device (1 =
 * no split; only shapes with at most 64 query rows per sequence split).
 * fa_split_workspace_bytes: bytes of `part` for num_splits (0 if < 2):
 * num_splits * B * Hq * Nq * (d + 1) * 4.
 * fa_fwd_kv_split: fa_fwd_kv with num_splits in [1, 256] (1 = plain
 * fa_fwd_kv; `part` may then be NULL); `part` is device memory of
 * fa_split_workspace_bytes() bytes, 16-byte aligned, clear of o and lse;
 * contents on entry do not matter.  16-bit inputs only (FA_ERR_DTYPE for
 * fp32).  Two launches (the split kernel, then the merge); allocates
 * nothing.
 * fa_fwd_kv_split_packed: the same with V packed by fa_pack_v.
 * fa_fwd and fa_fwd_kv never split. */
int fa_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int in_dtype);
size_t fa_split_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits);
int fa_fwd_kv_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_splits,
                    void* part, size_t part_bytes, void* stream, int in_dtype, int out_dtype);
int fa_fwd_kv_split_packed(const void* q, const void* k, const void* vt, size_t vt_bytes,
                           void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                           int causal, float scale, const int* cu_seqlens_q,
                           const int* cu_seqlens_k, int num_splits, void* part,
                           size_t part_bytes, void* stream, int in_dtype, int out_dtype);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fa_fwd_kv_split with the split-KV partials in a fixed device buffer the
 * library holds instead of a caller workspace.  Same results as
 * fa_fwd_kv_split with the same num_splits (the same kernels).  The buffer
 * is fa_noalloc_scratch_bytes() bytes (16 MiB) on each device the library
 * runs on, kept until the process ends; calls whose partials,
 * fa_split_workspace_bytes(B, Hq, Nq, d, num_splits), exceed it return
 * FA_ERR_SCRATCH before anything is enqueued.  Every call on one device
 * uses the same buffer, so calls that overlap in time on one device (other
 * streams, other threads) race: the caller serialises them.  Calls no
 * hipMalloc, hipFree or allocating library routine.  Other arguments and
 * errors as fa_fwd_kv_split. */
int fa_fwd_kv_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
                            int num_splits, void* stream, int in_dtype, int out_dtype);
size_t fa_noalloc_scratch_bytes(void);

/* Backward pass: the gradients dQ, dK, dV of sum(O * dO) for the forward of
 * fa_fwd (same B, Hq, Hkv, N, d, causal, scale, cu_seqlens and layouts).
 * The Kotaemon page calls the method tiling plus recomputation (the
 * paragraph after the formula): P is recomputed tile by tile from the
 * forward's lse instead of being stored, so no N x N matrix is kept.
 * With D_r = sum_j dO_rj O_rj:  dV = P^T dO,  dS = P * (dO V^T - D),
 * dQ = scale * dS K,  dK = scale * dS^T Q; a K/V head's gradients sum over
 * the query heads of its group.
 *
 * Inputs: q, k, v (in_dtype FA_F16 or FA_BF16), o (the forward's output in
 * o_dtype, FA_F32 or in_dtype), dout (in_dtype, o's layout), lse (fp32, as
 * written by the forward); scale finite and > 0 (FA_ERR_SCALE otherwise).
 * Outputs dq (q's layout), dk, dv (k's layout)
 * in grad_dtype (FA_F32 or in_dtype); they must not overlap any input, each
 * other or the workspace.  workspace: device memory of
 * fa_bwd_workspace_bytes() bytes, 16-byte aligned (the rows' D and
 * L * log2(e), fp32); contents on entry do not matter.  Allocates
 * nothing; errors as fa_fwd plus FA_ERR_WORKSPACE, FA_ERR_DTYPE for fp32
 * inputs. */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int in_dtype);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
           int causal, float scale, const int* cu_seqlens, void* workspace,
           size_t workspace_bytes, void* stream, int in_dtype, int o_dtype, int grad_dtype);

/* Block-sparse attention.  The Kotaemon page names block-sparse attention
 * only as a direction of the method (its closing outlook), with no layout;
 * the reading here: a 0/1 mask over blocks of 64 query rows x 64 keys
 * removes whole blocks of scores (set to -inf, as the causal mask removes
 * single scores); everything else is fa_fwd_kv.
 *
 * block_mask: DEVICE uint8 array [mask_batches][mask_heads][ceil(Nq/64)]
 * [ceil(Nk/64)], C order.  Entry (b, h, i, j) != 0 admits query rows
 * [64i, 64i+64) of sequence b, query head h against its keys [64j, 64j+64)
 * (row and key indices within the sequence, so for the packed layout each
 * sequence uses the top-left corner of its slab).  mask_batches is 1 (one
 * mask for every sequence) or B; mask_heads is 1 or Hq.  With causal = 1
 * the causal mask (bottom-right, as fa_fwd_kv) applies as well.  Rows that
 * see no key get O = 0 and L = -inf.  The mask must not overlap o or lse;
 * its size is not checked (the caller allocates mask_batches * mask_heads *
 * ceil(Nq/64) * ceil(Nk/64) bytes).
 *
 * 16-bit inputs only (FA_ERR_DTYPE for fp32); ceil(Nk/64) <= 4096 (keys per
 * sequence <= 262144, else FA_ERR_SHAPE); never split over keys; one launch,
 * no allocation.  fa_fwd_sparse_packed reads V packed by fa_pack_v (called
 * with N = Nk and cu_seqlens = cu_seqlens_k).  Other arguments and errors
 * as fa_fwd_kv. */
int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  const unsigned char* block_mask, int mask_batches, int mask_heads,
                  void* stream, int in_dtype, int out_dtype);
int fa_fwd_sparse_packed(const void* q, const void* k, const void* vt, size_t vt_bytes,
                         void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         int causal, float scale, const int* cu_seqlens_q,
                         const int* cu_seqlens_k, const unsigned char* block_mask,
                         int mask_batches, int mask_heads, void* stream, int in_dtype,
                         int out_dtype);

/* The argument checks of fa_fwd alone: returns what fa_fwd would return
 * before touching the device (FA_OK if it would go on to launch).  Makes no
 * HIP call, so it is usable without a GPU. */
int fa_fwd_check(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, int B, int Hq, int Hkv, int N, int d,
                 int causal, float scale, const int* cu_seqlens,
                 int in_dtype, int out_dtype);

/* Name of the kernel fa_fwd launches for these settings, or NULL if they are
 * unsupported.  Lets a caller confirm that this library, not a fallback, ran
 * (the Kotaemon page's caveats recommend checking that the fast attention
 * path is really active).  The string is static; do not free it.  This is
 * the kernel for query counts N with (Hq / Hkv) * N > 32; below that
 * fa_kernel_name_kv names the decode kernel that runs instead. */
const char* fa_kernel_name(int in_dtype, int d, int causal, int varlen,
                           int out_dtype);

/* Name of the kernel fa_fwd_kv (and fa_fwd, with Nq = N) launches for these
 * settings, head counts and query count Nq (the longest sequence's): for
 * 16-bit inputs with (Hq / Hkv) * Nq <= 32 the decode kernel, which packs
 * the query heads of a K/V head into one 32-row block, else as
 * fa_kernel_name.  NULL if unsupported (or Hkv < 1). */
const char* fa_kernel_name_kv(int in_dtype, int d, int causal, int varlen, int out_dtype,
                              int Hq, int Hkv, int Nq);

/* fa_kernel_name_kv for a given path: sparse = 1 for fa_fwd_sparse*,
 * vt_packed = 1 for the *_packed entry points (V packed by fa_pack_v). */
const char* fa_kernel_name_ex(int in_dtype, int d, int causal, int varlen, int out_dtype,
                              int Hq, int Hkv, int Nq, int sparse, int vt_packed);

/* The check FA_DEBUG=1 applies to a packed offset array, on HOST memory:
 * FA_OK if cu_seqlens[0] == 0 and 0 <= cu_seqlens[i] - cu_seqlens[i-1] <=
 * n_max for i = 1 .. B; FA_ERR_SEQLENS otherwise; FA_ERR_NULL for NULL and
 * FA_ERR_SHAPE for B < 0.  Makes no HIP call. */
int fa_check_seqlens(const int* cu_seqlens, int B, int n_max);

/* Testing aid for order independence (no counterpart on the pages: every
 * workgroup of the attention kernels writes only its own rows of O and L,
 * or of dQ, and reads only the inputs, so the order in which workgroups are
 * handed out must not change a single bit; a difference means a race).
 * Forces that order for the 16-bit forward kernels (fa_fwd, fa_fwd_kv,
 * fa_fwd_sparse, the split-KV and packed forms; not the decode kernel) and
 * for the dQ kernel of fa_bwd: -1 = the library's own choice (the default),
 * 0 = unit-major, 1 = unit-major with the XCD remap, 2 = row-block-major,
 * 3 = row-block-major with the XCD remap.  The remap applies only where the
 * launch allows it (the number of (sequence, head group) units a multiple
 * of 8, no KV split); the fp32 kernel, the decode kernel and the dK/dV
 * kernel keep their single order.  The initial value is FA_FORCE_ORDER from
 * the environment (the same numbers), else -1.  Process-wide; each launch
 * reads it once, so set it only while no launch is being prepared on
 * another thread.  Returns FA_OK, or FA_ERR_SHAPE for an order outside
 * -1 .. 3 (the setting is then unchanged).  Makes no HIP call. */
int fa_debug_force_order(int order);

/* The launch order currently forced (-1 .. 3, as fa_debug_force_order
 * takes it).  Makes no HIP call. */
int fa_debug_forced_order(void);

/* 1 if fa_fwd supports (in_dtype, d, causal), else 0 — so a caller can pick
 * another attention path when this one does not apply. */
int fa_supported(int in_dtype, int d, int causal);

/* Static description of a status code; never NULL. */
const char* fa_status_string(int status);

/* Build flags of this library: bit 0 (FA_BUILD_POISON_LDS) is set in the
 * LDS-poisoning test build (libfa_poison.so), whose kernels fill their LDS
 * with NaN before use so that a read of LDS they never wrote shows in the
 * result; the normal build returns 0.  Makes no HIP call. */
#define FA_BUILD_POISON_LDS 1
int fa_build_flags(void);

/* Library version as major*10000 + minor*100 + patch (the Kotaemon page's
 * caveats recommend pinning versions). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
