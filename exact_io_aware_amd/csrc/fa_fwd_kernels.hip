// Exact IO-aware attention forward ("FlashAttention") for gfx950 (MI355X).
//
// What is computed: O = softmax(scale * Q K^T) V and the per-row natural-log
// logsumexp L (the standard formula of the Kotaemon page, "Kotaemon
// FlashAttention应用：加快注意力计算", formula paragraph; L is the normaliser
// the tiling sketch of the HolySheep Flash Attention article, French edition,
// returns next to O).
//
// How (the method list of the Kotaemon page): Q is cut into row blocks; for
// each row block the K/V blocks are streamed through on-chip memory (LDS);
// each block's local dot products update a running row maximum and
// normaliser, the accumulated output is rescaled and the block's P.V added;
// O is normalised and written once at the end.  The score matrix never
// leaves registers.
//
// gfx950 mapping (our design, not the pages'):
//  * A workgroup is 8 waves (two per SIMD).  Each wave owns 32 query rows of
//    one query head.  For GQA, up to 4 query heads sharing a K/V head share
//    the workgroup, so one K/V tile in LDS feeds all of them.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//    the 32x32 accumulator puts one query per lane column (lane l and l+32
//    hold the same query), so the row max / row sum are in-lane except one
//    exchange between the two half-waves.
//  * The probabilities P^T stay in registers: the accumulator layout of
//    S^T is exactly the B-operand layout of O^T = V^T P^T once the key order
//    inside each 16-key chunk is permuted (0-3,8-11 | 4-7,12-15).  A small
//    pre-pass (fa_vt_pack) writes V^T tiles with the keys already in that
//    order, so the A operand is one 16-byte LDS read per lane.
//  * K and V^T tiles are double-buffered in LDS (one barrier per tile) and
//    filled straight from memory (buffer_load ... lds); loads of tile j+1
//    are in flight while tile j is computed.
//  * Online softmax in the log2 domain (scale*log2(e) folded into one FMA
//    per score), with the running maximum moved lazily: only when a row's
//    partial sum over a block leaves [0, 2^15].  The rescale is exact, so
//    the result is the same mathematically; most blocks skip the O rescale.
//  * Causal: tiles entirely above the diagonal are never visited; only
//    diagonal and ragged-tail blocks take the per-element mask.
//  * Row blocks run longest-first within each (sequence, head group), and
//    each (sequence, head group) runs on one XCD (workgroups are dealt
//    round-robin over the 8 XCDs), keeping its K/V in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

struct FwdParams {
  const void* q; const void* k; const void* v; void* o; float* lse;
  const int* cu_seqlens;   // query offsets (varlen)
  const int* cu_seqlens_k; // key/value offsets (varlen)
  int N, Nk, Hq, G;        // max query count, max key count, query heads, Hq / Hkv
  int hp, rows_per_wg, n_rblocks, n_hgroups, total_wg, xcd_remap;
  // rb_major (causal): row-block slot s of every unit is launched before slot
  // s + 1 of any, slot s being a sequence's s-th longest row block.
  int rb_major, n_units;
  float scale_log2;        // scale * log2(e)
  const void* vt;          // packed V^T tiles (16-bit inputs), see fa_vt_pack
  int Hkv, vt_ntiles;      // K/V heads; V^T tiles per (sequence, K/V head)
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

// LDS list of a block-sparse workgroup's key tiles (entry: tile index in
// the low 16 bits, one bit per wave that needs the tile above them) and
// per-wave counts for building it; a placeholder in the dense kernels.
template <bool SPARSE> struct SparseTiles { int e[kMaxSparseTiles]; int cnt[8]; };
template <> struct SparseTiles<false> { int e[1]; int cnt[1]; };
static_assert(kMaxSparseTiles <= 0xffff, "tile index in 16 bits");

// ---------------------------------------------------------------------------
// V^T packing: for every (sequence, K/V head, 64-key tile), write the tile
// transposed, D rows x 64 keys, keys in vt_key order, to the workspace:
// tile (b, kvh, t) at byte ((b * Hkv + kvh) * ntiles + t) * 128 * D.  Keys
// past the sequence end are zero.  Tiles wholly past it are not written (the
// attention kernel never reads them).
struct VtParams {
  const void* v; void* ws; const int* cu_seqlens;
  int N, Hkv, ntiles;
  long long kv_bs, kv_hs, kv_rs;
};

template <typename T, int D, bool VARLEN>
__global__ __launch_bounds__(256) void fa_vt_pack(VtParams p) {
  // One workgroup per tile: blockIdx.x = (b * Hkv + kvh) * ntiles + t.  The
  // tile's 64 V rows go straight into LDS (row-major, rm_swz layout; rows
  // past the sequence end read zeros); transposing LDS reads then give each
  // lane 8 keys of one column in exactly the V^T row order (the order of the
  // P.V operand), which it stores as one 16-byte chunk.
  constexpr int CPR = D / 8, RB = 2 * D, DB = D / 32;
  constexpr int LOADS = 64 * CPR / 256;
  const int t = blockIdx.x % p.ntiles;
  const int kvh = (blockIdx.x / p.ntiles) % p.Hkv;
  const int b = blockIdx.x / p.ntiles / p.Hkv;
  int seq0 = 0, len = p.N;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
  }
  const int kb = t * 64;
  if (kb >= len) return;
  __shared__ __attribute__((aligned(16))) char vl[64 * RB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const T* src = (const T*)p.v + (VARLEN ? (long long)seq0 * p.kv_rs : (long long)b * p.kv_bs) +
                 (long long)kvh * p.kv_hs + (long long)kb * p.kv_rs;
  const uint32_t rs_bytes = (uint32_t)p.kv_rs * 2;
  const int rows = __builtin_amdgcn_readfirstlane(min(64, len - kb));
  const rsrc_t r = make_rsrc(src, (uint32_t)rows * rs_bytes);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pch = tid + 256 * i;
    const int row = pch / CPR, pc = pch % CPR;
    lds_load16(r, vl + (256 * i + 64 * wave) * 16, row * rs_bytes + ((pc ^ rm_swz<D>(row)) << 4));
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // Pair (16-key group g, column block cb): lane L holds column 32 cb + L % 32,
  // positions 8 (L / 32) .. +7 of group g, i.e. chunk 2 g + L / 32 of that
  // V^T row.
  char* dst = (char*)p.ws + (long long)blockIdx.x * (128LL * D);
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int pair = wave + 4 * i;            // 4 * DB pairs over 4 waves
    const int g = pair & 3, cb = pair >> 2;
    const int tb = tr_base<D>(lane, cb);
    const u32x4 x = lds_read_tr<u32x4>(vl + tb + 16 * g * RB, vl + (tb ^ 32) + (16 * g + 8) * RB);
    *(u32x4*)(dst + (32 * cb + (lane & 31)) * 128 + (2 * g + (lane >> 5)) * 16) = x;
  }
}

// ---------------------------------------------------------------------------
// 16-bit (bf16 / fp16) inputs: MFMA kernel.
//
// Each wave owns QB blocks of 32 query rows of one head; every K or V operand
// it reads from LDS feeds the MFMAs of all QB blocks.  Keys are processed in
// 32-key blocks; K/V tiles of 64 keys (two blocks) are double-buffered in LDS.
// Step i of a wave masks block i if needed, issues the MFMAs of block i+1's
// scores, forms block i's probabilities (independent work, so the matrix
// cores and the vector ALUs overlap), then accumulates P.V of block i.
//
// SPARSE: a block mask removes whole 64 x 64 blocks of scores.  The
// workgroup streams only the key tiles that some wave's mask row admits, in
// key order; a wave whose own row does not admit a tile forms P = 0 for it.
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32, bool SPARSE>
__global__ __launch_bounds__(64 * waves_per_wg(FA_BF16, D, CAUSAL), 2) void fa_fwd_mfma(FwdParams p) {
  using vec8 = typename Ops<T>::vec8;
  constexpr int NW = waves_per_wg(FA_BF16, D, CAUSAL);  // waves per workgroup
  constexpr int NT = 64 * NW;                      // threads per workgroup
  constexpr int QB = rows_per_wave(FA_BF16) / 32;  // 32-row query blocks per wave
  constexpr int WR = 32 * QB;                // query rows per wave
  constexpr int BC = 64;                     // keys per K/V tile (two 32-key blocks)
  constexpr int DB = D / 32;                 // 32-wide blocks of the output
  constexpr int DC = D / 16;                 // 16-wide chunks of Q.K
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per tile row
  constexpr int LOADS = BC * CPR / NT;       // 16-byte loads per thread per tile
  constexpr int TILE_BYTES = BC * RB;
  constexpr int HALF = 32 * RB;              // bytes of one 32-key block in a tile

  // Two LDS buffers per operand, as separate objects so that reads of one
  // are known not to alias the direct-to-LDS loads landing in the other.
  __shared__ __attribute__((aligned(16))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds1[TILE_BYTES];
  __shared__ SparseTiles<SPARSE> sp;
  static_assert(!SPARSE || NW <= 8, "one list bit per wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hf = lane >> 5;

  // a1: workgroup -> (unit = sequence b x head group, row block).
  // Workgroups are dealt round-robin over the 8 XCDs (workgroup j on XCD
  // j % 8).  With xcd_remap, XCD x takes the units u with u % 8 == x, each
  // unit's row blocks consecutively: all row blocks of a unit (which share
  // its K/V) stay in one XCD's L2, and every XCD gets an equal share of
  // every sequence, whatever the sequence lengths.
  int wg = blockIdx.x, split = 0;
  if (p.n_splits > 1) {                      // consecutive workgroups: splits of one unit
    split = wg % p.n_splits;
    wg /= p.n_splits;
  }
  //
  // Under the causal mask row blocks differ in length.  Dispatched
  // unit by unit, the last units' long row blocks start when most CUs are
  // already busy, and they set the launch's end; with rb_major the
  // longest row blocks of all units go first (each unit still on its XCD)
  // and the short ones fill the tail.
  const int idx = p.xcd_remap ? wg >> 3 : wg;
  const int nu = p.xcd_remap ? p.n_units >> 3 : p.n_units;  // units in this order
  int k, rb;
  if (p.rb_major) {
    rb = idx / nu;
    k = idx - rb * nu;
  } else {
    k = idx / p.n_rblocks;
    rb = idx - k * p.n_rblocks;
  }
  const int unit = p.xcd_remap ? 8 * k + (wg & 7) : k;
  const int b = unit / p.n_hgroups;
  const int hgrp = unit - b * p.n_hgroups;
  const int h = hgrp * p.hp + (wave % p.hp);
  const int kvh = (hgrp * p.hp) / p.G;

  // Query rows [0, len) and keys [0, len_k) of sequence b.  The queries are
  // the last len tokens of the sequence: with the causal mask, row r sees
  // keys c <= r + off, off = len_k - len.
  int seq0 = 0, len = p.N, seq0_k = 0, len_k = p.Nk;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
    seq0_k = p.cu_seqlens_k[b];
    len_k = p.cu_seqlens_k[b + 1] - seq0_k;
  }
  // Longest row blocks first: under the causal mask those are the last
  // ones of the sequence (slot s is row block nrb - 1 - s).
  if (CAUSAL) rb = (VARLEN ? (len + p.rows_per_wg - 1) / p.rows_per_wg : p.n_rblocks) - 1 - rb;
  const int off = len_k - len;
  const int wg_row0 = rb * p.rows_per_wg;
  if (rb < 0 || wg_row0 >= len) return;      // uniform over the workgroup
  const int row0 = wg_row0 + (wave / p.hp) * WR;
  const int wg_rows_end = min(wg_row0 + p.rows_per_wg, len);
  const int kv_end = CAUSAL ? max(0, min(wg_rows_end + off, len_k)) : len_k;
  const bool active = row0 < len;
  const int wave_kv_end = CAUSAL ? max(0, min(min(row0 + WR, len) + off, len_k)) : len_k;
  const int wave_nblk = active ? (wave_kv_end + 31) / 32 : 0;  // blocks this wave needs
  // This workgroup's key tiles: [t_begin, t_begin + split_tiles) (all of
  // them without split-KV); blk0 is the first 32-key block.
  const int t_begin = split * p.split_tiles;
  const int kv_stop = min(kv_end, (t_begin + p.split_tiles) * BC);
  const int blk0 = 2 * t_begin;
  // Blocks this wave softmaxes: its own, and none past the split's range
  // (their P.V would belong to the next split).
  const int wave_blk_end = min(wave_nblk, (kv_stop + 31) / 32);

  const long long qbase = (VARLEN ? (long long)seq0 * p.q_rs : (long long)b * p.q_bs) +
                          (long long)h * p.q_hs;
  const long long kvbase = (VARLEN ? (long long)seq0_k * p.kv_rs : (long long)b * p.kv_bs) +
                           (long long)kvh * p.kv_hs;
  const char* kp = (const char*)((const T*)p.k + kvbase);
  const uint32_t kv_rs_bytes = (uint32_t)p.kv_rs * 2;

  // Block-sparse: list the key tiles some wave needs, in key order.  Wave w
  // (head hgrp*hp + w%hp, rows from r0) needs tile j if the mask row of its
  // 64-row query block admits j and, with the causal mask, the tile starts
  // before the wave's last visible key.  Each thread tests one tile; a
  // ballot and the per-wave counts place the admitted tiles.
  int n_list = 0;
  if constexpr (SPARSE) {
    const int ntk = (kv_end + BC - 1) / BC;
    const uint8_t* mb = p.block_mask + p.mask_bs * b;
    for (int base = 0; base < ntk; base += NT) {
      const int j = base + tid;
      uint32_t bits = 0;
      if (j < ntk) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int r0 = wg_row0 + (w / p.hp) * WR;
          const int hw = hgrp * p.hp + (w % p.hp);
          const int kend = CAUSAL ? min(min(r0 + WR, len) + off, len_k) : len_k;
          if (r0 < len && j * BC < kend &&
              mb[p.mask_hs * hw + (long long)(r0 / kSparseBlock) * p.mask_nkb + j] != 0)
            bits |= 1u << w;
        }
      }
      const uint64_t bal = __ballot(bits != 0);
      if (lane == 0) sp.cnt[wave] = (int)__popcll(bal);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = sp.cnt[w];
        before += w < wave ? c : 0;
        total += c;
      }
      if (bits != 0)
        sp.e[n_list + before + (int)__popcll(bal & ((1ull << lane) - 1ull))] =
            j | (int)(bits << 16);
      n_list += total;
      __syncthreads();
    }
    n_list = __builtin_amdgcn_readfirstlane(n_list);
  }
  // The tile streamed at position pos, as a list entry: dense, the tile
  // index; sparse, the list entry (past the list, a tile past every
  // sequence end with no wave bits: it reads zeros and is never softmaxed).
  // The sparse loop reads the entries it needs once per iteration, right
  // after a barrier, when no other LDS read is waiting.
  auto entry = [&](int pos) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) {
      const int e = __builtin_amdgcn_readfirstlane(sp.e[min(pos, kMaxSparseTiles - 1)]);
      return pos < n_list ? e : p.vt_ntiles;
    } else {
      return t_begin + pos;
    }
  };
  auto tile_of = [&](int e) __attribute__((always_inline)) -> int {
    return SPARSE ? (e & 0xffff) : e;
  };
  // Key block i of the streamed sequence (half i % 2 of the tile whose entry
  // is e): its first key, and whether this wave softmaxes it (a block past
  // the wave's keys or, sparse, outside its mask row gets P = 0).
  auto blk = [&](int i, int e, int& kb, bool& live) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      kb = (e & 0xffff) * BC + 32 * (i & 1);
      live = ((e >> (16 + wave)) & 1) != 0 && kb < wave_kv_end;
    } else {
      kb = (blk0 + i) * 32;
      live = blk0 + i < wave_blk_end;
    }
  };

  // a3: tile loads go straight from memory into LDS (buffer_load ... lds):
  // lane L of wave w in load i fills 16-byte LDS chunk position
  // q = NT*i + 64*w + L of the tile, i.e. row q / CPR, position q % CPR,
  // which holds the row's chunk (q % CPR) ^ swizzle(row).  Rows past the
  // sequence end (and whole tiles past it) read zeros.
  uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pch = tid + NT * i;
    const int r = pch / CPR, pc = pch % CPR;
    koff[i] = r * kv_rs_bytes + ((pc ^ k_swz<D>(r)) << 4);
    const int vr = pch / 8, vc = pch % 8;       // V^T tile: 8 chunks per row
    voff[i] = vr * 128 + ((vc ^ vt_swz(vr)) << 4);
  }
  auto gload = [&](int e, char* dst_base) __attribute__((always_inline)) {
    const int kb = tile_of(e) * BC;
    // readfirstlane keeps the clamp (a VALU med3) in a scalar register: the
    // resource of a buffer load must be wave-uniform.
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(len_k - kb, BC)));
    const rsrc_t r = make_rsrc(kp + (long long)min(kb, len_k) * kv_rs_bytes,
                               (uint32_t)rows * kv_rs_bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) lds_load16(r, dst_base + (NT * i + 64 * wave) * 16, koff[i]);
  };
  const char* vtp = (const char*)p.vt + (long long)(b * p.Hkv + kvh) * p.vt_ntiles * TILE_BYTES;
  auto gload_vt = [&](int e, char* dst_base) __attribute__((always_inline)) {
    // A V^T tile is contiguous; tiles past the sequence end read zeros.
    const int tile = tile_of(e);
    const int live_tile = __builtin_amdgcn_readfirstlane(tile * BC < len_k ? 1 : 0);
    const rsrc_t r = make_rsrc(vtp + (long long)min(tile, p.vt_ntiles) * TILE_BYTES,
                               live_tile ? (uint32_t)TILE_BYTES : 0u);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) lds_load16(r, dst_base + (NT * i + 64 * wave) * 16, voff[i]);
  };

  // Prologue loads: K_0, K_1 and V_0 (K runs ahead of V).
  gload(entry(0), k_lds0);
  gload_vt(entry(0), v_lds0);
  gload(entry(1), k_lds1);

  // a2: this wave's Q rows as MFMA B operands (query block qb, d-chunk dc,
  // 8 values per lane: Q[row0 + 32*qb + l32][16*dc + 8*hf .. +7]).  Rows past
  // the end read zeros; their results are never stored.
  vec8 qf[QB][DC];
  {
    const int qrows = __builtin_amdgcn_readfirstlane(active ? min(WR, len - row0) : 0);
    const rsrc_t rq = make_rsrc((const T*)p.q + qbase + (long long)(active ? row0 : 0) * p.q_rs,
                                (uint32_t)qrows * (uint32_t)p.q_rs * 2);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t qo = (uint32_t)((32 * qb + l32) * p.q_rs + hf * 8) * 2;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        qf[qb][dc] = __builtin_bit_cast(
            vec8, __builtin_amdgcn_raw_buffer_load_b128(rq, qo + dc * 32, 0, 0));
    }
  }

  // Per-lane LDS byte offsets of the MFMA operand reads; everything else in
  // those addresses is a compile-time constant (an instruction offset).
  //  K (A operand of S^T = K Q^T): block row l32, chunk 2*dc + hf.
  int kaddr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) kaddr[dc] = l32 * RB + (((2 * dc + hf) ^ k_swz<D>(l32)) << 4);
  //  V^T (A operand of O^T = V^T P^T): output block db, row 32*db + l32; for
  //  key half hb of the tile and 16-key chunk kc, logical chunk 4*hb + 2*kc + hf
  //  (8 keys in vt_key order).  Index [2*hb + kc]; db is an instruction offset.
  int vaddr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) vaddr[q] = l32 * 128 + (((2 * q + hf) ^ vt_swz(l32)) << 4);

  f32x16 oacc[QB][DB];
  float m_run[QB], ell[QB];         // reference maximum (log2 units), partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[qb][i] = f32x16{};
    m_run[qb] = kNoMax;
    ell[qb] = 0.0f;
  }
  const float sl2 = p.scale_log2;

  // a4: S^T = K Q^T for one 32-key block (rows of `ks`), every query block.
  auto qk = [&](const char* ks, f32x16 (&s)[QB]) __attribute__((always_inline)) {
    vec8 kf[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kf[dc] = *(const vec8*)(ks + kaddr[dc]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = Ops<T>::mfma(kf[dc], qf[qb][dc], s[qb]);
  };

  // a5: masks of the 32-key block from key kb, only where it crosses the
  // diagonal or the end of the sequence.
  auto mask = [&](int kb, f32x16 (&s)[QB]) __attribute__((always_inline)) {
    if ((CAUSAL && kb + 31 > row0 + off) || (kb + 32 > len_k)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + 8 * (e >> 2) + 4 * hf + (e & 3);
          if ((CAUSAL && key > row0 + 32 * qb + l32 + off) || key >= len_k)
            s[qb][e] = -__builtin_inff();
        }
    }
  };

  // a6: online softmax of one block.  P is formed against the reference
  // maximum m (form_p); if a lane's partial sum leaves [0, 2^15] (a score far
  // above m, or the first block, where m = -inf), m moves to the true running
  // maximum, O and ell are rescaled by exp2(m_old - m_new) and P is formed
  // again (settle).  The rescale is exact, so the result does not depend on
  // when m moves.
  //
  // The block's row sum: with bf16 P (8 significant bits) it is taken from
  // the fp32 P, as a tree of adds (short dependency chains); with fp16 P it
  // is taken from the rounded P itself, two values per v_dot2 (relative
  // error at most 2^-11 per value, so L moves by at most ~4.9e-4, and O is
  // the exact mean of V under the weights the P.V product uses).
  auto form_p = [&](const f32x16 (&s)[QB], uint32_t (&pk)[QB][8], float (&lsum)[QB],
                    bool live) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // A block past the wave's last one gets m = +inf: P = 0 and sum 0.
      const float m = live ? m_run[qb] : __builtin_inff();
      float t[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][e], sl2, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][e + 1], sl2, -m));
        pk[qb][e >> 1] = Ops<T>::pack(p0, p1);
        if constexpr (!Ops<T>::kSumRounded) t[e >> 1] = p0 + p1;
      }
      if constexpr (Ops<T>::kSumRounded) {
        float a = 0.0f, c = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          a = Ops<T>::sum2(pk[qb][j], a);
          c = Ops<T>::sum2(pk[qb][j + 1], c);
        }
        lsum[qb] = a + c;
      } else {
        lsum[qb] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
      }
    }
  };
  auto settle = [&](const f32x16 (&s)[QB], uint32_t (&pk)[QB][8], float (&lsum)[QB])
      __attribute__((always_inline)) {
    bool ok = true;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ok = ok && (lsum[qb] <= kSumLimit);
    if (__any(!ok)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][e]);
        // mx = -inf only for rows with no visible key yet, which keep kNoMax.
        const float m_new = fmaxf(m_run[qb], halves_max(mx) * sl2);
        const float alpha = m_new == m_run[qb] ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        ell[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
        m_run[qb] = m_new;
      }
      form_p(s, pk, lsum, true);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ell[qb] += lsum[qb];
  };

  // a7: O^T += V^T P^T over the two 16-key chunks of one block: key half hb
  // of the V^T tile at vs.
  auto pv = [&](const char* vs, int hb, const uint32_t (&pk)[QB][8])
      __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      vec8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        u32x4 pb = {pk[qb][4 * kc + 0], pk[qb][4 * kc + 1], pk[qb][4 * kc + 2], pk[qb][4 * kc + 3]};
        pf[qb] = __builtin_bit_cast(vec8, pb);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const vec8 vf = *(const vec8*)(vs + vaddr[2 * hb + kc] + db * 32 * 128);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = Ops<T>::mfma(vf, pf[qb], oacc[qb][db]);
      }
    }
  };

  // Step s of the three-stage pipeline: scores of block s+1 (MFMA), softmax
  // of block s (VALU) and P.V of block s-1 (MFMA) are independent, so they
  // are issued together and the matrix cores and vector ALUs overlap.  The
  // same straight-line code serves every step: past a wave's last block its
  // P is zero (and its scores, reads of loaded or zero-filled LDS, unused),
  // so the step after the last one just drains P.V.
  auto step = [&](int st, int e_st, f32x16 (&s_cur)[QB], f32x16 (&s_nxt)[QB],
                  uint32_t (&pk_cur)[QB][8], const uint32_t (&pk_prev)[QB][8],
                  const char* ks_nxt, const char* vs_prev, int hb_prev)
      __attribute__((always_inline)) {
    // A wave with no rows (past the sequence end: a partial last row block,
    // or the empty row groups of a decode step) only takes part in the
    // loads and barriers.
    if (!active) return;
    int kb;
    bool live;
    blk(st, e_st, kb, live);
    mask(kb, s_cur);
    float lsum[QB];
    qk(ks_nxt, s_nxt);
    form_p(s_cur, pk_cur, lsum, live);
    pv(vs_prev, hb_prev, pk_prev);
    // Issue order for the region above: a few operand reads ahead, then each
    // MFMA (32 cycles in the matrix pipe) followed by a few independent
    // softmax instructions and the next reads, so the wave's exp/FMA work
    // runs while its own MFMAs execute.
    // d = 64 has half the MFMAs per block for the same softmax work, so
    // more vector instructions go with each MFMA.
    constexpr int QK_VALU = D == 128 ? 2 : 5, QK_LDS = 2;
    constexpr int PV_VALU = D == 128 ? 3 : 6;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // 4 LDS reads
#pragma unroll
    for (int i = 0; i < DC * QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // 1 MFMA (scores)
      __builtin_amdgcn_sched_group_barrier(0x002, QK_VALU, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, QK_LDS, 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * DB * QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // 1 MFMA (P.V)
      __builtin_amdgcn_sched_group_barrier(0x002, PV_VALU, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // 1 LDS read
    }
    settle(s_cur, pk_cur, lsum);
  };

  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // K_0, K_1, V_0 and Q have landed
  __syncthreads();
  f32x16 sA[QB], sB[QB];
  uint32_t pkA[QB][8], pkB[QB][8];
  qk(k_lds0, sA);
  {                                  // step 0: no P.V yet
    float lsum[QB];
    int kb0;
    bool live0;
    blk(0, entry(0), kb0, live0);
    mask(kb0, sA);
    qk(k_lds0 + HALF, sB);
    form_p(sA, pkA, lsum, live0);
    settle(sA, pkA, lsum);
  }
  // Barrier B_t follows step 2t: all of K_t and V_{t-1} have been read, so
  // K_{t+2} and V_{t+1} start streaming into their buffers; every step reads
  // data that landed at least one barrier earlier.  Loads past the last tile
  // fetch nothing and write zeros.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  gload(entry(2), k_lds0);
  gload_vt(entry(1), v_lds1);

  // Steps 1 .. nblk (the last one drains P.V), four per iteration so that
  // every buffer is a fixed object: K_t sits in k_lds[t % 2], V_t in
  // v_lds[t % 2]; step s reads K of block s+1 and V of block s-1.
  const int last_step = SPARSE ? 2 * n_list : max(0, (kv_stop + 31) / 32 - blk0);
  for (int u = 0; 4 * u + 1 <= last_step; ++u) {
    const int s1 = 4 * u + 1;
    // Steps s1 .. s1+3 softmax blocks of tiles 2u (second half), 2u+1 and
    // 2u+2 (first half); this iteration loads K of tiles 2u+3, 2u+4 and V
    // of tiles 2u+2, 2u+3.
    const int e0 = entry(2 * u), e1 = entry(2 * u + 1), e2 = entry(2 * u + 2);
    const int e3 = entry(2 * u + 3), e4 = entry(2 * u + 4);
    step(s1, e0, sB, sA, pkB, pkA, k_lds1, v_lds0, 0);
    if (s1 + 1 > last_step) break;
    step(s1 + 1, e1, sA, sB, pkA, pkB, k_lds1 + HALF, v_lds0, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    gload(e3, k_lds1);
    gload_vt(e2, v_lds0);
    if (s1 + 2 > last_step) break;
    step(s1 + 2, e1, sB, sA, pkB, pkA, k_lds0, v_lds1, 0);
    if (s1 + 3 > last_step) break;
    step(s1 + 3, e2, sA, sB, pkA, pkB, k_lds0 + HALF, v_lds1, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    gload(e4, k_lds0);
    gload_vt(e3, v_lds1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no load left in flight
  // Every wave has finished reading K/V from LDS: the tile buffers become
  // the epilogue's staging area.
  __syncthreads();
  if (!active) return;

  if (p.n_splits > 1) {
    // Split-KV partial: this split's normalised O and L (O = 0, L = -inf
    // where the split holds no visible key); a merge pass combines splits.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float ell_t = halves_sum(ell[qb]);
      const float inv = ell_t > 0.0f ? 1.0f / ell_t : 0.0f;
      const int qrow = row0 + 32 * qb + l32;
      if (qrow < len) {
        const long long prow = (((long long)split * p.B + b) * p.Hq + h) * p.N + qrow;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *(f32x4*)(p.o_part + prow * D + 32 * db + 8 * g4 + 4 * hf) =
                f32x4{oacc[qb][db][4 * g4] * inv, oacc[qb][db][4 * g4 + 1] * inv,
                      oacc[qb][db][4 * g4 + 2] * inv, oacc[qb][db][4 * g4 + 3] * inv};
        if (hf == 0) p.lse_part[prow] = (m_run[qb] + __builtin_amdgcn_logf(ell_t)) * kLn2;
      }
    }
    return;
  }

  // a8: epilogue.  O = acc / ell, L = (m + log2 ell) * ln 2.
  //
  // The accumulator gives each lane one query row and scattered 16-byte
  // pieces of it, so stores straight from registers would touch 32 rows per
  // instruction.  Each wave instead stages its rows in its share of the four
  // tile buffers (SLOT bytes: 8 KiB at d = 128, 4 KiB at d = 64), DBP
  // output blocks of 32 columns at a time, and stores whole row segments
  // (consecutive lanes write consecutive 16-byte chunks of a row).
  using OT = typename std::conditional<OUT_F32, float, T>::type;
  constexpr int OB = sizeof(OT);
  constexpr int SLOT = 4 * TILE_BYTES / NW;          // staging bytes per wave
  constexpr int PER_BUF = TILE_BYTES / SLOT;         // staging slots per tile buffer
  static_assert(NW % 4 == 0 && PER_BUF * SLOT == TILE_BYTES, "staging slots");
  constexpr int DBP = (DB < SLOT / (32 * 32 * OB)) ? DB : SLOT / (32 * 32 * OB);
  constexpr int RP = DBP * 32 * OB;                  // staged bytes per row
  constexpr int CPO = RP / 16;                       // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPO;                      // rows per store instruction
  static_assert(DBP >= 1 && DB % DBP == 0 && 32 * RP <= SLOT, "staging slot size");
  const int sbuf = wave / PER_BUF;
  char* slot = sbuf == 0 ? k_lds0 : sbuf == 1 ? k_lds1 : sbuf == 2 ? v_lds0 : v_lds1;
  slot += (wave % PER_BUF) * SLOT;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ell_t = halves_sum(ell[qb]);
    // A row that sees no key (causal, more queries than keys) has ell = 0:
    // O = 0 and L = -inf.
    const float inv = ell_t > 0.0f ? 1.0f / ell_t : 0.0f;
    const int qrow = row0 + 32 * qb + l32;
    if (hf == 0 && qrow < len) {
      const long long li = ((long long)b * p.Hq + h) * p.N + qrow;
      p.lse[li] = (m_run[qb] + __builtin_amdgcn_logf(ell_t)) * kLn2;
    }
#pragma unroll
    for (int pass = 0; pass < DB / DBP; ++pass) {
      // Stage: lane (l32, hf) holds row l32, columns 32*db + 8*g4 + 4*hf + 0..3.
#pragma unroll
      for (int j = 0; j < DBP; ++j) {
        const int db = pass * DBP + j;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float a0 = oacc[qb][db][4 * g4 + 0] * inv, a1 = oacc[qb][db][4 * g4 + 1] * inv;
          const float a2 = oacc[qb][db][4 * g4 + 2] * inv, a3 = oacc[qb][db][4 * g4 + 3] * inv;
          if (OUT_F32) {
            const int c = 8 * j + 2 * g4 + hf;
            *(f32x4*)(slot + l32 * RP + ((c ^ (l32 & (CPO - 1))) << 4)) = f32x4{a0, a1, a2, a3};
          } else {
            const int c = 4 * j + g4;
            u32x2 w = {Ops<T>::pack(a0, a1), Ops<T>::pack(a2, a3)};
            *(u32x2*)(slot + l32 * RP + ((c ^ (l32 & (CPO - 1))) << 4) + 8 * hf) = w;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the wave's own writes landed
      // Store: lane L takes chunk L % CPO of row it*RPI + L / CPO.
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int r = it * RPI + lane / CPO, c = lane % CPO;
        const u32x4 v = *(const u32x4*)(slot + r * RP + ((c ^ (r & (CPO - 1))) << 4));
        const int orow_i = row0 + 32 * qb + r;
        if (orow_i < len) {
          char* dst = (char*)((OT*)p.o + qbase + (long long)orow_i * p.q_rs) + pass * RP + c * 16;
          // O is written once and not read back here: a non-temporal store
          // (whole row segments) keeps it from displacing K/V in the caches.
          __builtin_nontemporal_store(v, (u32x4*)dst);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // reads done before the slot is rewritten
    }
  }
}

// ---------------------------------------------------------------------------
// Decode: few query rows per sequence (G * nq <= 32) against a long key /
// value cache.  The G query heads of a K/V head and their nq rows form one
// 32-row MFMA block (packed row r = hh * nq + i: head g * G + hh, query i),
// so one wave covers the whole group for the keys it streams, and the
// workgroup's 4 waves (one per SIMD, with the whole register file) share
// out the unit's 64-key tiles (wave w takes tiles w, w + 4, ...).  The work
// is HBM-bound, so the loads are built for bandwidth: each wave reads its
// tiles (32 KiB: 64 K rows and the packed V^T tile, both contiguous) with
// 1 KiB non-temporal loads into registers, one tile ahead, and passes each
// tile through its own LDS slot to put it in the MFMA operand layouts; no
// workgroup barrier inside the loop.  Per 32-key block: S^T =
// K Q^T (Q shared in LDS), the lazy online softmax of fa_fwd_mfma, O^T +=
// V^T P^T.  At the end the waves' (m, l, O) states are merged through LDS.
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void fa_decode_mfma(FwdParams p) {
  using vec8 = typename Ops<T>::vec8;
  constexpr int NW = 4;
  constexpr int DB = D / 32, DC = D / 16, CPR = D / 8, RB = D * 2;
  constexpr int TILE_BYTES = 64 * RB;        // 64 K rows, or one packed V^T tile
  constexpr int STAGE = 2 * TILE_BYTES;      // K rows then V^T
  constexpr int LOADS = STAGE / 1024;        // 1 KiB loads per tile
  constexpr int OS = D + 4;                  // floats per staged O row
  static_assert(NW * 32 * OS * 4 <= NW * STAGE, "merge area fits the slots");
  // One tile per wave; after the loop, the waves' O.
  __shared__ __attribute__((aligned(16))) char slots[NW * STAGE];
  __shared__ __attribute__((aligned(16))) char q_lds[32 * RB];
  __shared__ float m_s[NW][32], l_s[NW][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;

  int wg = blockIdx.x, split = 0;
  if (p.n_splits > 1) {
    split = wg % p.n_splits;
    wg /= p.n_splits;
  }
  const int b = wg / p.Hkv;
  const int g = wg - b * p.Hkv;
  int seq0 = 0, len = p.N, seq0_k = 0, len_k = p.Nk;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
    seq0_k = p.cu_seqlens_k[b];
    len_k = p.cu_seqlens_k[b + 1] - seq0_k;
  }
  if (len <= 0) return;                      // uniform: no rows
  const int nrows = p.G * len;               // packed rows in use (<= 32)
  const int off = len_k - len;               // row i sees keys c <= i + off

  // Tiles of this workgroup: [t0, t0 + ntl), 64 keys each (the split range
  // starts on a tile; keys at or past k_stop are masked).
  const int t0 = split * p.split_tiles;
  const int k_stop = min(len_k, (split + 1) * p.split_tiles * 64);
  const int ntl = max(0, (k_stop - 64 * t0 + 63) / 64);
  const int my_tiles = ntl > wave ? (ntl - wave + NW - 1) / NW : 0;   // wave-uniform

  const long long kvbase = (VARLEN ? (long long)seq0_k * p.kv_rs : (long long)b * p.kv_bs) +
                           (long long)g * p.kv_hs;
  const uint32_t kv_rs_bytes = (uint32_t)p.kv_rs * 2;
  const char* kp = (const char*)((const T*)p.k + kvbase);
  const char* vtp = (const char*)p.vt + (long long)(b * p.Hkv + g) * p.vt_ntiles * TILE_BYTES;

  // Q block into LDS: thread t fills rows t / CPR (+ 256 / CPR), chunk
  // t % CPR, with rm_swz (zeros past the group's nrows).
  for (int q = tid; q < 32 * CPR; q += NW * 64) {
    const int rr = q / CPR, c = q % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rr < nrows) {
      const int hh = rr / len, i = rr - hh * len;
      const long long qo = (VARLEN ? (long long)(seq0 + i) * p.q_rs
                                   : (long long)b * p.q_bs + (long long)i * p.q_rs) +
                           (long long)(g * p.G + hh) * p.q_hs + 8 * c;
      v = *(const u32x4*)((const T*)p.q + qo);
    }
    *(u32x4*)(q_lds + rr * RB + ((c ^ rm_swz<D>(rr)) << 4)) = v;
  }
  __syncthreads();                           // Q block written

  // The cache is read once per call: non-temporal loads (cache policy NT),
  // which stream through the caches at a higher HBM rate than ordinary
  // loads (measured on MI355X: ~7.1 against ~6.0 TB/s for a plain read).
  constexpr int kNT = 2;
  // Tile j of the wave in registers: load i brings 1 KiB chunk i (lane L:
  // bytes 16 L of it), first the 64 K rows (row r = position / CPR, chunk
  // pc), then the V^T tile (row vr = position / 8 of 128 B, chunk vc).
  // Rows past the sequence end, and tiles past the wave's last, read zeros
  // (bounded buffers); the loads are issued unconditionally so every path
  // keeps the same loads in flight.
  struct Stage { u32x4 x[LOADS]; };
  auto gload = [&](int j, Stage& st) __attribute__((always_inline)) {
    const int t = t0 + wave + NW * j;
    const int kb = 64 * t;
    const bool in = j < my_tiles;
    const int rows = __builtin_amdgcn_readfirstlane(in ? max(0, min(len_k - kb, 64)) : 0);
    const rsrc_t rk = make_rsrc(kp + (long long)min(kb, len_k) * kv_rs_bytes,
                                (uint32_t)rows * kv_rs_bytes);
    const rsrc_t rv = make_rsrc(vtp + (long long)(in ? t : 0) * TILE_BYTES,
                                in ? (uint32_t)TILE_BYTES : 0u);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = 64 * i + lane;
      if (i < TILE_BYTES / 1024) {
        const int r = q / CPR, pc = q % CPR;
        st.x[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, r * kv_rs_bytes + 16 * pc, 0, kNT));
      } else {
        st.x[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * (q - TILE_BYTES / 16), 0, kNT));
      }
    }
  };
  // ... and into the wave's LDS slot, swizzled for the operand reads: K
  // chunk pc of row r at position pc ^ k_swz(r) (rows of RB bytes); V^T
  // chunk vc of row vr at vc ^ vt_swz(vr) (rows of 128 bytes).
  char* const my_slot = slots + wave * STAGE;
  auto swrite = [&](const Stage& st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = 64 * i + lane;
      if (i < TILE_BYTES / 1024) {
        const int r = q / CPR, pc = q % CPR;
        *(u32x4*)(my_slot + r * RB + ((pc ^ k_swz<D>(r)) << 4)) = st.x[i];
      } else {
        const int qv = q - TILE_BYTES / 16;
        const int vr = qv >> 3, vc = qv & 7;
        *(u32x4*)(my_slot + TILE_BYTES + vr * 128 + ((vc ^ vt_swz(vr)) << 4)) = st.x[i];
      }
    }
  };

  // This lane's packed row (the S^T accumulator column): query qi of head
  // g * G + (l32 / len); rows past nrows compute on zero Q and are never
  // stored.
  const int qi = l32 - (l32 / len) * len;
  const float sl2 = p.scale_log2;
  // Read offsets: Q^T chunk dc (B operand, row l32, chunk 2 dc + hf), K
  // chunk dc (A operand, row 32 h + l32 of the tile, chunk 2 dc + hf), V^T
  // row 32 db + l32, keys chunk 4 h + 2 kc + hf.
  const int qaddr0 = l32 * RB + ((hf ^ rm_swz<D>(l32)) << 4);
  const int kaddr0 = l32 * RB + ((hf ^ k_swz<D>(l32)) << 4);
  const int vaddr0 = TILE_BYTES + l32 * 128 + ((hf ^ vt_swz(l32)) << 4);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = kNoMax, ell = 0.0f;

  // Key block h (32 keys from kb) of the tile in the slot.
  auto compute = [&](int kb, int h) __attribute__((always_inline)) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const vec8 kf = *(const vec8*)(my_slot + 32 * h * RB + (kaddr0 ^ (32 * dc)));
      const vec8 qf = *(const vec8*)(q_lds + (qaddr0 ^ (32 * dc)));
      s = Ops<T>::mfma(kf, qf, s);
    }
    // Mask where the block crosses the sequence end or (causal) the first
    // row's last visible key.
    if (kb + 32 > len_k || (CAUSAL && kb + 31 > off)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (key >= len_k || (CAUSAL && key > qi + off)) s[e] = -__builtin_inff();
      }
    }
    // Lazy online softmax, as in fa_fwd_mfma (P against the reference
    // maximum; move it only when a lane's partial sum leaves [0, 2^15]).
    uint32_t pk[8];
    float lsum;
    auto form = [&]() __attribute__((always_inline)) {
      float t[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sl2, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + 1], sl2, -m_run));
        pk[e >> 1] = Ops<T>::pack(p0, p1);
        t[e >> 1] = p0 + p1;
      }
      lsum = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    };
    form();
    if (__any(!(lsum <= kSumLimit))) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      const float m_new = fmaxf(m_run, halves_max(mx) * sl2);
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      ell *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      m_run = m_new;
      form();
    }
    ell += lsum;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 pb = {pk[4 * kc], pk[4 * kc + 1], pk[4 * kc + 2], pk[4 * kc + 3]};
      const vec8 pf = __builtin_bit_cast(vec8, pb);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const vec8 vf = *(const vec8*)(my_slot + db * 32 * 128 + (vaddr0 ^ (32 * (2 * h + kc))));
        oacc[db] = Ops<T>::mfma(vf, pf, oacc[db]);
      }
    }
  };

  // Tile j + 1 loads into the registers while tile j, written to the slot,
  // is computed (its second half only when it holds keys before k_stop).
  Stage st;
  gload(0, st);
  for (int j = 0; j < my_tiles; ++j) {
    swrite(st);
    gload(j + 1, st);
    const int kb = 64 * (t0 + wave + NW * j);
    compute(kb, 0);
    if (kb + 32 < k_stop) compute(kb + 32, 1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));        // the trailing (zero) loads

  // Merge the waves: each stages its O^T (fp32, row l32, columns
  // 32 db + 8 g4 + 4 hf + 0..3), m and l per row; the slots are free once
  // every wave has left the loop.
  const float ell_t = halves_sum(ell);
  __syncthreads();
  auto ostage = [&](int w) __attribute__((always_inline)) -> float* {
    return (float*)slots + w * 32 * OS;
  };
  float* const os_me = ostage(wave);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *(f32x4*)(os_me + l32 * OS + 32 * db + 8 * g4 + 4 * hf) =
          f32x4{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
  if (hf == 0) {
    m_s[wave][l32] = m_run;
    l_s[wave][l32] = ell_t;
  }
  __syncthreads();
  // Thread t: row t / 8, columns (t % 8) * D / 8 ..: L = M + log2 l,
  // O = sum_w 2^(m_w - M) O_w / l, with M the largest m_w (a wave that saw
  // no key of the row has l_w = 0 and adds nothing).
  constexpr int CW = D / 8;
  const int rr = tid >> 3, c0 = (tid & 7) * CW;
  if (rr >= nrows) return;
  float M = kNoMax;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, m_s[w][rr]);
  float wt[NW], l = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = l_s[w][rr] > 0.0f ? __builtin_amdgcn_exp2f(m_s[w][rr] - M) : 0.0f;
    l += wt[w] * l_s[w][rr];
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float ov[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) ov[c] = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int c = 0; c < CW; c += 4) {
      const f32x4 x = *(const f32x4*)(ostage(w) + rr * OS + c0 + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) ov[c + u] += wt[w] * x[u];
    }
  const int hh = rr / len, i = rr - hh * len;
  if (i >= p.N) return;                      // (a sequence longer than N: not stored)
  const int h = g * p.G + hh;
  const float lse_row = l > 0.0f ? (M + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff();
  if (p.n_splits > 1) {
    const long long prow = (((long long)split * p.B + b) * p.Hq + h) * p.N + i;
#pragma unroll
    for (int c = 0; c < CW; c += 4)
      *(f32x4*)(p.o_part + prow * D + c0 + c) =
          f32x4{ov[c] * inv, ov[c + 1] * inv, ov[c + 2] * inv, ov[c + 3] * inv};
    if ((tid & 7) == 0) p.lse_part[prow] = lse_row;
    return;
  }
  const long long qbase = (VARLEN ? (long long)seq0 * p.q_rs : (long long)b * p.q_bs) +
                          (long long)h * p.q_hs + (long long)i * p.q_rs + c0;
  using OT = typename std::conditional<OUT_F32, float, T>::type;
  OT* dst = (OT*)p.o + qbase;
#pragma unroll
  for (int c = 0; c < CW; c += 4) {
    if (OUT_F32) {
      *(f32x4*)((float*)dst + c) = f32x4{ov[c] * inv, ov[c + 1] * inv, ov[c + 2] * inv, ov[c + 3] * inv};
    } else {
      *(u32x2*)(dst + c) = u32x2{Ops<T>::pack(ov[c] * inv, ov[c + 1] * inv),
                                 Ops<T>::pack(ov[c + 2] * inv, ov[c + 3] * inv)};
    }
  }
  if ((tid & 7) == 0) p.lse[((long long)b * p.Hq + h) * p.N + i] = lse_row;
}

// ---------------------------------------------------------------------------
// Split-KV merge.  Each split s of a row holds O_s (normalised over its keys)
// and L_s = ln(sum of its exp-scores); the row's result is
//   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s,
// the same normaliser algebra as the online softmax, applied once.  32
// lanes per row, D/32 columns each; a row no split saw gives O = 0, L = -inf.
template <typename OT, int D, bool VARLEN>
__global__ __launch_bounds__(256) void fa_merge_splits(FwdParams p) {
  constexpr int PER = D / 32;
  const int row_id = blockIdx.x * 8 + (threadIdx.x >> 5);     // (b, h, r) flattened
  const int c0 = (threadIdx.x & 31) * PER;
  if (row_id >= p.B * p.Hq * p.N) return;
  const int r = row_id % p.N;
  const int bh = row_id / p.N;
  const int h = bh % p.Hq, b = bh / p.Hq;
  int seq0 = 0, len = p.N;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
  }
  if (r >= len) return;
  const long long stride = (long long)p.B * p.Hq * p.N;       // rows per split
  float lmax = -__builtin_inff();
  for (int s = 0; s < p.n_splits; ++s) lmax = fmaxf(lmax, p.lse_part[s * stride + row_id]);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  float wsum = 0.0f;
  if (lmax != -__builtin_inff()) {
    for (int s = 0; s < p.n_splits; ++s) {
      const float w = __expf(p.lse_part[s * stride + row_id] - lmax);
      wsum += w;
      const float* src = p.o_part + (s * stride + row_id) * D + c0;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += w * src[j];
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const long long orow = (VARLEN ? (long long)(seq0 + r) * p.q_rs : (long long)b * p.q_bs +
                                                                        (long long)r * p.q_rs) +
                         (long long)h * p.q_hs;
  OT* dst = (OT*)p.o + orow + c0;
#pragma unroll
  for (int j = 0; j < PER; ++j) dst[j] = (OT)(acc[j] * inv);
  if ((threadIdx.x & 31) == 0)
    p.lse[((long long)b * p.Hq + h) * p.N + r] = wsum > 0.0f ? lmax + __logf(wsum) : lmax;
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_32x32x2_f32 (full fp32 products and sums), P kept
// in fp32.  Same transposed formulation; one 32-key tile at a time.  Each
// wave owns 32 query rows; 4 waves cover 128 rows of one head.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fa_fwd_f32(FwdParams p) {
  constexpr int BC = 32;
  constexpr int KP = D + 1;      // padded K row (floats): conflict-free column reads
  constexpr int DB = D / 32;
  constexpr int DK = D / 2;      // k-steps of Q.K (2 per MFMA)
  __shared__ float ks[BC * KP];
  __shared__ float vs[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int unit = blockIdx.x / p.n_rblocks;
  int rb = blockIdx.x - unit * p.n_rblocks;
  if (CAUSAL) rb = p.n_rblocks - 1 - rb;
  const int b = unit / p.Hq;
  const int h = unit - b * p.Hq;
  const int kvh = h / p.G;
  int seq0 = 0, len = p.N, seq0_k = 0, len_k = p.Nk;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
    seq0_k = p.cu_seqlens_k[b];
    len_k = p.cu_seqlens_k[b + 1] - seq0_k;
  }
  const int off = len_k - len;                // row r sees keys c <= r + off (causal)
  const int wg_row0 = rb * 128;
  if (wg_row0 >= len) return;
  const int row0 = wg_row0 + wave * 32;
  const int kv_end = CAUSAL ? max(0, min(min(wg_row0 + 128, len) + off, len_k)) : len_k;
  const int ntiles = (kv_end + BC - 1) / BC;
  const bool active = row0 < len;
  const int wave_kv_end = CAUSAL ? max(0, min(min(row0 + 32, len) + off, len_k)) : len_k;
  const int wave_ntiles = active ? (wave_kv_end + BC - 1) / BC : 0;

  const long long qbase = (VARLEN ? (long long)seq0 * p.q_rs : (long long)b * p.q_bs) +
                          (long long)h * p.q_hs;
  const long long kvbase = (VARLEN ? (long long)seq0_k * p.kv_rs : (long long)b * p.kv_bs) +
                           (long long)kvh * p.kv_hs;
  const float* qp = (const float*)p.q + qbase;
  const float* kp = (const float*)p.k + kvbase;
  const float* vp = (const float*)p.v + kvbase;

  const int qrow = row0 + l32;
  float qf[DK];  // Q[qrow][2*t + hf]
  {
    const float* src = qp + (long long)min(qrow, len - 1) * p.q_rs;
#pragma unroll
    for (int t = 0; t < DK; ++t) qf[t] = src[2 * t + hf];
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNoMax, ell = 0.0f;

  // K/V tile j + 1 is fetched into registers while tile j is computed, so
  // each tile's HBM round trip overlaps the previous tile's work.  Element
  // e = tid + 256 i of a tile is row e / D, column e % D (rows past the end
  // repeat the last key; their scores are masked).
  constexpr int PER_T = BC * D / 256;
  float kpre[PER_T], vpre[PER_T];
  auto fetch = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int e = tid + 256 * i, r = e / D, c = e % D;
      const long long row = (long long)min(j * BC + r, len_k - 1) * p.kv_rs;
      kpre[i] = kp[row + c];
      vpre[i] = vp[row + c];
    }
  };
  if (ntiles > 0) fetch(0);
  for (int j = 0; j < ntiles; ++j) {
    const int kb = j * BC;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int e = tid + 256 * i, r = e / D, c = e % D;
      ks[r * KP + c] = kpre[i];
      vs[r * D + c] = vpre[i];
    }
    __syncthreads();
    if (j + 1 < ntiles) fetch(j + 1);
    if (j < wave_ntiles) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < DK; ++t)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * KP + 2 * t + hf], qf[t], s, 0, 0, 0);
      const bool need_mask = (CAUSAL && kb + BC - 1 > row0 + off) || (kb + BC > len_k);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if ((CAUSAL && key > qrow + off) || key >= len_k) s[i] = -__builtin_inff();
        }
      }
      // Online softmax against the reference maximum, moved (with an exact
      // rescale) when a partial sum leaves [0, 2^15]; see the 16-bit kernel.
      float pr[16], lsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -m_run));
        lsum += pr[i];
      }
      if (__any(!(lsum <= kSumLimit))) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float m_new = fmaxf(m_run, halves_max(mx) * p.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        ell *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = m_new;
        lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, -m_run));
          lsum += pr[i];
        }
      }
      ell += lsum;
      // O^T += V^T P^T: step i pairs key(i, half 0) and key(i, half 1).
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + 32 * db + l32], pr[i],
                                                         oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const float ell_t = halves_sum(ell);
  const float inv = ell_t > 0.0f ? 1.0f / ell_t : 0.0f;   // no visible key: O = 0
  if (qrow < len) {
    float* orow = (float*)p.o + qbase + (long long)qrow * p.q_rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        *(f32x4*)(orow + d0) = f32x4{oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                     oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
      }
    if (hf == 0)
      p.lse[((long long)b * p.Hq + h) * p.N + qrow] = (m_run + __builtin_amdgcn_logf(ell_t)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Dispatch table.
typedef void (*KernelFn)(FwdParams);

struct Variant {
  int in_dtype, d, causal, varlen, out_dtype, sparse;
  KernelFn fn;
  const char* name;
};

#define FA_SFX_C_0 ""
#define FA_SFX_C_1 "_causal"
#define FA_SFX_V_0 ""
#define FA_SFX_V_1 "_varlen"
#define FA_SFX_O_0 ""
#define FA_SFX_O_1 "_of32"
#define FA_CAT(a, b) a##b
#define FA_SFX_S_0 ""
#define FA_SFX_S_1 "_sparse"
#define FA_V16(T, TN, DT, D, C, VL, OF, SP)                                        \
  {DT, D, C, VL, (OF) ? FA_F32 : DT, SP,                                           \
   fa_fwd_mfma<T, D, (C != 0), (VL != 0), (OF != 0), (SP != 0)>,                   \
   "fa_fwd_mfma_" TN "_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)           \
       FA_CAT(FA_SFX_O_, OF) FA_CAT(FA_SFX_S_, SP)}
#define FA_V16_ALL(T, TN, DT, D, SP)                                              \
  FA_V16(T, TN, DT, D, 0, 0, 0, SP), FA_V16(T, TN, DT, D, 0, 0, 1, SP),            \
  FA_V16(T, TN, DT, D, 0, 1, 0, SP), FA_V16(T, TN, DT, D, 0, 1, 1, SP),            \
  FA_V16(T, TN, DT, D, 1, 0, 0, SP), FA_V16(T, TN, DT, D, 1, 0, 1, SP),            \
  FA_V16(T, TN, DT, D, 1, 1, 0, SP), FA_V16(T, TN, DT, D, 1, 1, 1, SP)
#define FA_V32(D, C, VL)                                                           \
  {FA_F32, D, C, VL, FA_F32, 0, fa_fwd_f32<D, (C != 0), (VL != 0)>,                \
   "fa_fwd_f32_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)}

const Variant kVariants[] = {
    FA_V16_ALL(__bf16, "bf16", FA_BF16, 64, 0), FA_V16_ALL(__bf16, "bf16", FA_BF16, 128, 0),
    FA_V16_ALL(_Float16, "f16", FA_F16, 64, 0), FA_V16_ALL(_Float16, "f16", FA_F16, 128, 0),
    FA_V16_ALL(__bf16, "bf16", FA_BF16, 64, 1), FA_V16_ALL(__bf16, "bf16", FA_BF16, 128, 1),
    FA_V16_ALL(_Float16, "f16", FA_F16, 64, 1), FA_V16_ALL(_Float16, "f16", FA_F16, 128, 1),
    FA_V32(64, 0, 0), FA_V32(64, 0, 1), FA_V32(64, 1, 0), FA_V32(64, 1, 1),
    FA_V32(128, 0, 0), FA_V32(128, 0, 1), FA_V32(128, 1, 0), FA_V32(128, 1, 1),
};

// Decode kernels (16-bit inputs, G * Nq <= 32).
struct DecodeVariant {
  int in_dtype, d, causal, varlen, out_dtype;
  KernelFn fn;
  const char* name;
};
#define FA_VD(T, TN, DT, D, C, VL, OF)                                            \
  {DT, D, C, VL, (OF) ? FA_F32 : DT, fa_decode_mfma<T, D, (C != 0), (VL != 0), (OF != 0)>, \
   "fa_decode_mfma_" TN "_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)          \
       FA_CAT(FA_SFX_O_, OF)}
#define FA_VD_ALL(T, TN, DT, D)                                                   \
  FA_VD(T, TN, DT, D, 0, 0, 0), FA_VD(T, TN, DT, D, 0, 0, 1),                      \
  FA_VD(T, TN, DT, D, 0, 1, 0), FA_VD(T, TN, DT, D, 0, 1, 1),                      \
  FA_VD(T, TN, DT, D, 1, 0, 0), FA_VD(T, TN, DT, D, 1, 0, 1),                      \
  FA_VD(T, TN, DT, D, 1, 1, 0), FA_VD(T, TN, DT, D, 1, 1, 1)
const DecodeVariant kDecodeVariants[] = {
    FA_VD_ALL(__bf16, "bf16", FA_BF16, 64), FA_VD_ALL(__bf16, "bf16", FA_BF16, 128),
    FA_VD_ALL(_Float16, "f16", FA_F16, 64), FA_VD_ALL(_Float16, "f16", FA_F16, 128),
};
const DecodeVariant* find_decode(int in_dtype, int d, int causal, int varlen, int out_dtype) {
  for (const DecodeVariant& v : kDecodeVariants)
    if (v.in_dtype == in_dtype && v.d == d && v.causal == causal && v.varlen == varlen &&
        v.out_dtype == out_dtype)
      return &v;
  return nullptr;
}

const Variant* find_variant(int in_dtype, int d, int causal, int varlen, int out_dtype,
                            int sparse = 0) {
  for (const Variant& v : kVariants)
    if (v.in_dtype == in_dtype && v.d == d && v.causal == causal && v.varlen == varlen &&
        v.out_dtype == out_dtype && v.sparse == sparse)
      return &v;
  return nullptr;
}

}  // namespace

typedef void (*PackFn)(VtParams);
struct PackVariant {
  int in_dtype, d, varlen;
  PackFn fn;
};
const PackVariant kPackVariants[] = {
    {FA_BF16, 64, 0, fa_vt_pack<__bf16, 64, false>}, {FA_BF16, 64, 1, fa_vt_pack<__bf16, 64, true>},
    {FA_BF16, 128, 0, fa_vt_pack<__bf16, 128, false>}, {FA_BF16, 128, 1, fa_vt_pack<__bf16, 128, true>},
    {FA_F16, 64, 0, fa_vt_pack<_Float16, 64, false>}, {FA_F16, 64, 1, fa_vt_pack<_Float16, 64, true>},
    {FA_F16, 128, 0, fa_vt_pack<_Float16, 128, false>}, {FA_F16, 128, 1, fa_vt_pack<_Float16, 128, true>},
};

typedef void (*MergeFn)(FwdParams);
struct MergeVariant {
  int out_dtype, d, varlen;
  MergeFn fn;
};
const MergeVariant kMergeVariants[] = {
    {FA_F32, 64, 0, fa_merge_splits<float, 64, false>},
    {FA_F32, 64, 1, fa_merge_splits<float, 64, true>},
    {FA_F32, 128, 0, fa_merge_splits<float, 128, false>},
    {FA_F32, 128, 1, fa_merge_splits<float, 128, true>},
    {FA_BF16, 64, 0, fa_merge_splits<__bf16, 64, false>},
    {FA_BF16, 64, 1, fa_merge_splits<__bf16, 64, true>},
    {FA_BF16, 128, 0, fa_merge_splits<__bf16, 128, false>},
    {FA_BF16, 128, 1, fa_merge_splits<__bf16, 128, true>},
    {FA_F16, 64, 0, fa_merge_splits<_Float16, 64, false>},
    {FA_F16, 64, 1, fa_merge_splits<_Float16, 64, true>},
    {FA_F16, 128, 0, fa_merge_splits<_Float16, 128, false>},
    {FA_F16, 128, 1, fa_merge_splits<_Float16, 128, true>},
};
MergeFn find_merge(int out_dtype, int d, bool varlen) {
  for (const MergeVariant& m : kMergeVariants)
    if (m.out_dtype == out_dtype && m.d == d && m.varlen == (int)varlen) return m.fn;
  return nullptr;
}

const char* kernel_name(int in_dtype, int d, int causal, int varlen, int out_dtype) {
  const Variant* v = find_variant(in_dtype, d, causal != 0, varlen != 0, out_dtype);
  return v ? v->name : nullptr;
}

const char* kernel_name_kv(int in_dtype, int d, int causal, int varlen, int out_dtype, int Hq,
                           int Hkv, int Nq) {
  if (use_decode(in_dtype, Hq, Hkv, Nq, false)) {
    const DecodeVariant* v = find_decode(in_dtype, d, causal != 0, varlen != 0, out_dtype);
    return v ? v->name : nullptr;
  }
  return kernel_name(in_dtype, d, causal, varlen, out_dtype);
}

int launch_fwd(const LaunchArgs& a, void* stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  const bool sparse = a.block_mask != nullptr;
  if (sparse && a.in_dtype == FA_F32) return FA_ERR_DTYPE;
  const Variant* var = find_variant(a.in_dtype, a.d, a.causal, varlen, a.out_dtype, sparse);
  if (!var) return FA_ERR_DTYPE;
  const bool decode = use_decode(a.in_dtype, a.Hq, a.Hkv, a.N, sparse);
  const DecodeVariant* dvar = decode ? find_decode(a.in_dtype, a.d, a.causal, varlen, a.out_dtype)
                                     : nullptr;
  if (decode && !dvar) return FA_ERR_DTYPE;
  const Plan plan = make_plan(a.B, a.Hq, a.Hkv, a.N, a.d, a.in_dtype, a.causal);

  FwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
  p.cu_seqlens = a.cu_seqlens; p.cu_seqlens_k = a.cu_seqlens_k;
  p.N = a.N; p.Nk = a.Nk; p.Hq = a.Hq; p.G = a.Hq / a.Hkv;
  p.hp = plan.hp; p.rows_per_wg = plan.rows_per_wg; p.n_rblocks = plan.n_rblocks;
  p.n_hgroups = plan.n_hgroups; p.total_wg = (int)plan.total_wg;
  p.xcd_remap = (a.in_dtype != FA_F32) && ((uint64_t)a.B * plan.n_hgroups) % 8 == 0;
  p.n_units = a.B * plan.n_hgroups;
  p.scale_log2 = a.scale * kLog2e;
  p.vt = a.vt; p.Hkv = a.Hkv; p.vt_ntiles = vt_tiles(a.Nk);
  const int n_splits = (a.in_dtype != FA_F32 && !sparse && a.n_splits > 1) ? a.n_splits : 1;
  p.n_splits = n_splits;
  // Row-block-major order pays when the launch is a few rounds of
  // workgroups deep (at most 4 per resident slot): then unit-major order
  // starts the last units' long row blocks late and they set the launch's
  // end.  With more rounds unit-major is already close to longest-first,
  // and it keeps one unit's K/V at a time in the XCD's L2, where
  // row-block-major spreads each XCD over all its units (more L2 misses).
  // It also needs all K/V (the largest sequence length for every sequence)
  // to fit in half of the 256 MB last-level cache, else each unit's K/V
  // re-reads by its row blocks go to HBM.
  p.rb_major = 0;
  if (a.causal && !decode && 4LL * a.B * a.Hkv * a.Nk * a.d <= (128LL << 20)) {
    int dev = -1, cus = 0, per_cu = 0;
    const int threads = 64 * waves_per_wg(a.in_dtype, a.d, a.causal);
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)var->fn, threads, 0) ==
            hipSuccess &&
        cus > 0 && per_cu > 0)
      p.rb_major = plan.total_wg * (uint64_t)n_splits <= 4ull * (uint64_t)cus * (uint64_t)per_cu;
  }
  p.split_tiles = n_splits > 1 ? (p.vt_ntiles + n_splits - 1) / n_splits : p.vt_ntiles + 1;
  p.B = a.B; p.o_part = a.o_part; p.lse_part = a.lse_part;
  p.block_mask = a.block_mask;
  p.mask_nkb = (a.Nk + kSparseBlock - 1) / kSparseBlock;
  {
    const long long slab = (long long)((a.N + kSparseBlock - 1) / kSparseBlock) * p.mask_nkb;
    p.mask_hs = a.mask_heads > 1 ? slab : 0;
    p.mask_bs = a.mask_batches > 1 ? slab * a.mask_heads : 0;
  }
  if (n_splits > 1) p.xcd_remap = 0;
  const long long d = a.d;
  if (varlen) {
    p.q_bs = 0; p.q_hs = d; p.q_rs = (long long)a.Hq * d;
    p.kv_bs = 0; p.kv_hs = d; p.kv_rs = (long long)a.Hkv * d;
  } else {
    p.q_rs = d; p.q_hs = (long long)a.N * d; p.q_bs = (long long)a.Hq * a.N * d;
    p.kv_rs = d; p.kv_hs = (long long)a.Nk * d; p.kv_bs = (long long)a.Hkv * a.Nk * d;
  }
  void* args[] = {&p};
  // Decode: one 4-wave workgroup per (sequence, K/V head, split).
  const hipError_t e =
      decode ? hipLaunchKernel((const void*)dvar->fn,
                               dim3((unsigned)((uint64_t)a.B * a.Hkv * (uint64_t)n_splits)),
                               dim3(256), args, 0, (hipStream_t)stream)
             : hipLaunchKernel((const void*)var->fn,
                               dim3((unsigned)(plan.total_wg * (uint64_t)n_splits)),
                               dim3(64 * waves_per_wg(a.in_dtype, a.d, a.causal)), args, 0,
                               (hipStream_t)stream);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  if (n_splits == 1) return FA_OK;
  const MergeFn mf = find_merge(a.out_dtype, a.d, varlen);
  if (!mf) return FA_ERR_DTYPE;
  const uint64_t rows = (uint64_t)a.B * a.Hq * a.N;
  const hipError_t e2 = hipLaunchKernel((const void*)mf, dim3((unsigned)((rows + 7) / 8)),
                                        dim3(256), args, 0, (hipStream_t)stream);
  return e2 == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int suggest_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int in_dtype, int cus) {
  if (in_dtype == FA_F32 || Nq > 64 || cus <= 0) return 1;
  // The 8-wave plan (a causal d = 64 launch has up to twice the
  // workgroups, of half the size).
  const Plan plan = make_plan(B, Hq, Hkv, Nq, d, in_dtype, false);
  // One workgroup fills a compute unit (its eight waves take the VGPRs of
  // two per SIMD, and the decode kernel's merge area most of the LDS); split
  // only grids smaller than one per compute unit.
  const uint64_t want = (uint64_t)cus;
  const uint64_t wgs = use_decode(in_dtype, Hq, Hkv, Nq, false) ? (uint64_t)B * Hkv : plan.total_wg;
  if (wgs >= want) return 1;
  const int tiles = vt_tiles(Nk);
  uint64_t n = (want + wgs - 1) / wgs;
  const uint64_t max_by_len = (uint64_t)tiles / 4;     // at least 4 tiles (256 keys) a split
  if (n > max_by_len) n = max_by_len;
  if (n > 64) n = 64;
  return n < 1 ? 1 : (int)n;
}

int launch_vt_pack(const void* v, void* vt, int B, int Hkv, int N, int d, const int* cu_seqlens,
                   int in_dtype, void* stream) {
  const int varlen = cu_seqlens != nullptr;
  const PackVariant* var = nullptr;
  for (const PackVariant& pv : kPackVariants)
    if (pv.in_dtype == in_dtype && pv.d == d && pv.varlen == varlen) var = &pv;
  if (!var) return FA_ERR_DTYPE;
  VtParams p;
  p.v = v; p.ws = vt; p.cu_seqlens = cu_seqlens;
  p.N = N; p.Hkv = Hkv; p.ntiles = vt_tiles(N);
  if (varlen) {
    p.kv_bs = 0; p.kv_hs = d; p.kv_rs = (long long)Hkv * d;
  } else {
    p.kv_rs = d; p.kv_hs = (long long)N * d; p.kv_bs = (long long)Hkv * N * d;
  }
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel((const void*)var->fn,
                                       dim3((unsigned)((long long)B * Hkv * p.ntiles)), dim3(256),
                                       args, 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
