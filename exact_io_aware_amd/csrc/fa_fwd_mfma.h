// The MFMA attention kernel for 16-bit inputs (bf16 / fp16): exact IO-aware
// attention forward ("FlashAttention") on gfx950 (MI355X).
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
//    inside each 16-key chunk is permuted (0-3,8-11 | 4-7,12-15).  The A
//    operand V^T comes from the row-major V tile in LDS through two
//    transposing reads (ds_read_b64_tr_b16), which deliver the keys in
//    exactly that order; or, for V packed beforehand by fa_vt_pack (the
//    decode cache's layout), from one 16-byte read.
//  * K and V tiles are double-buffered in LDS (one barrier per tile) and
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
#ifndef FA_FWD_MFMA_H
#define FA_FWD_MFMA_H

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_fwd_common.h"
#include "fa_internal.h"
#include "fa_poison.h"

namespace fa {
namespace {

// the low 16 bits, one bit per wave that needs the tile above them) and
// per-wave counts for building it; a placeholder in the dense kernels.
template <bool SPARSE> struct SparseTiles { int e[kMaxSparseTiles]; int cnt[8]; };
template <> struct SparseTiles<false> { int e[1]; int cnt[1]; };
static_assert(kMaxSparseTiles <= 0xffff, "tile index in 16 bits");

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
//
// VPACK: V comes as packed V^T tiles (fa_vt_pack; the decode cache's
// layout) instead of the row-major V.
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32, bool SPARSE, bool VPACK>
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
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(k_lds0, TILE_BYTES, tid, NT);
    poison_lds(k_lds1, TILE_BYTES, tid, NT);
    poison_lds(v_lds0, TILE_BYTES, tid, NT);
    poison_lds(v_lds1, TILE_BYTES, tid, NT);
    __syncthreads();
  }

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
  const char* vp = (const char*)((const T*)p.v + kvbase);
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
  // which holds the row's chunk (q % CPR) ^ rm_swz(row).  K and V tiles
  // share that row-major layout (conflict-free both for the reads by rows
  // of K and for the transposing reads of V).  Rows past the sequence end
  // (and whole tiles past it) read zeros.
  uint32_t koff[LOADS], voff[VPACK ? LOADS : 1];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pch = tid + NT * i;
    const int r = pch / CPR, pc = pch % CPR;
    koff[i] = r * kv_rs_bytes + ((pc ^ rm_swz<D>(r)) << 4);
    if constexpr (VPACK) {
      const int vr = pch / 8, vc = pch % 8;     // V^T tile: 8 chunks per row
      voff[i] = vr * 128 + ((vc ^ vt_swz(vr)) << 4);
    }
  }
  // Rows [kb, kb + 64) of the K (or V) rows at `base` into a tile buffer.
  auto gload_rows = [&](const char* base, int e, char* dst_base) __attribute__((always_inline)) {
    const int kb = tile_of(e) * BC;
    // readfirstlane keeps the clamp (a VALU med3) in a scalar register: the
    // resource of a buffer load must be wave-uniform.
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(len_k - kb, BC)));
    const rsrc_t r = make_rsrc(base + (long long)min(kb, len_k) * kv_rs_bytes,
                               (uint32_t)rows * kv_rs_bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) lds_load16(r, dst_base + (NT * i + 64 * wave) * 16, koff[i]);
  };
  auto gload = [&](int e, char* dst_base) __attribute__((always_inline)) {
    gload_rows(kp, e, dst_base);
  };
  const char* vtp = (const char*)p.vt + (long long)(b * p.Hkv + kvh) * p.vt_ntiles * TILE_BYTES;
  auto gload_vt = [&](int e, char* dst_base) __attribute__((always_inline)) {
    if constexpr (VPACK) {
      // A V^T tile is contiguous; tiles past the sequence end read zeros.
      const int tile = tile_of(e);
      const int live_tile = __builtin_amdgcn_readfirstlane(tile * BC < len_k ? 1 : 0);
      const rsrc_t r = make_rsrc(vtp + (long long)min(tile, p.vt_ntiles) * TILE_BYTES,
                                 live_tile ? (uint32_t)TILE_BYTES : 0u);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_load16(r, dst_base + (NT * i + 64 * wave) * 16, voff[i]);
    } else {
      gload_rows(vp, e, dst_base);
    }
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
  for (int dc = 0; dc < DC; ++dc) kaddr[dc] = l32 * RB + (((2 * dc + hf) ^ rm_swz<D>(l32)) << 4);
  //  V^T (A operand of O^T = V^T P^T), output block db.  Packed V^T: row
  //  32*db + l32; for key half hb of the tile and 16-key chunk kc, logical
  //  chunk 4*hb + 2*kc + hf (8 keys in vt_key order), index [2*hb + kc]; db
  //  is an instruction offset.  Row-major V: two transposing reads per
  //  operand (rows 16*(2*hb + kc) .. +7 and +8 .. +15 of the tile), at the
  //  lane offsets vtr[db] and vtr2[db] = (vtr[db] ^ 32) (the second half's
  //  swizzle differs in one chunk bit).
  int vaddr[VPACK ? 4 : 1], vtr[VPACK ? 1 : DB], vtr2[VPACK ? 1 : DB];
  if constexpr (VPACK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) vaddr[q] = l32 * 128 + (((2 * q + hf) ^ vt_swz(l32)) << 4);
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      vtr[db] = tr_base<D>(lane, db);
      vtr2[db] = vtr[db] ^ 32;
    }
  }

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
  // of the V (or packed V^T) tile at vs.  pv_read fetches the block's V^T
  // operands (chunk kc, output block db), pv_mma issues its MFMAs.
  auto pv_read = [&](const char* vs, int hb, vec8 (&vf)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (VPACK) {
          vf[kc][db] = *(const vec8*)(vs + vaddr[2 * hb + kc] + db * 32 * 128);
        } else {
          const int r0 = 32 * hb + 16 * kc;
          vf[kc][db] = lds_read_tr<vec8>(vs + vtr[db] + r0 * RB, vs + vtr2[db] + (r0 + 8) * RB);
        }
      }
  };
  auto pv_mma = [&](const vec8 (&vf)[2][DB], const uint32_t (&pk)[QB][8])
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
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = Ops<T>::mfma(vf[kc][db], pf[qb], oacc[qb][db]);
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
    // Past the step that drains the wave's last block (causal: a wave's
    // rows end before its workgroup's) there is nothing left to add.
    if constexpr (!SPARSE) {
      if (blk0 + st - 1 >= wave_blk_end) return;
    }
    int kb;
    bool live;
    blk(st, e_st, kb, live);
    mask(kb, s_cur);
    float lsum[QB];
    vec8 vf[2][DB];
    if constexpr (D == 64) {
      // d = 64: every V^T operand of the step is read first and the
      // compiler orders the rest (its own order measured 3-4 % faster on
      // causal d = 64 than the issue groups below, which serve d = 128).
      pv_read(vs_prev, hb_prev, vf);
      qk(ks_nxt, s_nxt);
      form_p(s_cur, pk_cur, lsum, live);
      pv_mma(vf, pk_prev);
      settle(s_cur, pk_cur, lsum);
      return;
    }
    qk(ks_nxt, s_nxt);
    form_p(s_cur, pk_cur, lsum, live);
    pv_read(vs_prev, hb_prev, vf);
    pv_mma(vf, pk_prev);
    // Issue order for the region above: a few operand reads ahead, then each
    // MFMA (32 cycles in the matrix pipe) followed by a few independent
    // softmax instructions and the next reads, so the wave's exp/FMA work
    // runs while its own MFMAs execute (d = 128).
    constexpr int QK_VALU = 2, QK_LDS = 2;
    constexpr int PV_VALU = 3;
    constexpr int PV_LDS = VPACK ? 1 : 2;           // operand reads per P.V MFMA
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
      __builtin_amdgcn_sched_group_barrier(0x100, PV_LDS, 0);
    }
    settle(s_cur, pk_cur, lsum);
  };

  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // K_0, K_1, V_0 and Q have landed
  __syncthreads();
  // A scale <= 0 enters through Q (negated for scale < 0, zero for scale =
  // 0) with |scale| (or 1) in scale_log2, so scores and masks keep their
  // positive-scale form.  Wave-uniform; exact.
  if (p.q_mode != 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 x = __builtin_bit_cast(u32x4, qf[qb][dc]);
        const uint32_t sgn = 0x80008000u;
        qf[qb][dc] = __builtin_bit_cast(
            vec8, p.q_mode == 1 ? u32x4{x[0] ^ sgn, x[1] ^ sgn, x[2] ^ sgn, x[3] ^ sgn}
                                : u32x4{0u, 0u, 0u, 0u});
      }
  }
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

}  // namespace
}  // namespace fa

// The instance table of one (input type, head dimension): every causal /
// varlen / fp32-O / sparse / packed-V combination, and the function that
// returns it.
#define FA_SFX_C_0 ""
#define FA_SFX_C_1 "_causal"
#define FA_SFX_V_0 ""
#define FA_SFX_V_1 "_varlen"
#define FA_SFX_O_0 ""
#define FA_SFX_O_1 "_of32"
#define FA_SFX_S_0 ""
#define FA_SFX_S_1 "_sparse"
#define FA_SFX_P_0 ""
#define FA_SFX_P_1 "_vtpacked"
#define FA_CAT(a, b) a##b
#define FA_V16(T, TN, DT, D, C, VL, OF, SP, VP)                                    \
  {DT, D, C, VL, (OF) ? FA_F32 : DT, SP, VP,                                       \
   fa::fa_fwd_mfma<T, D, (C != 0), (VL != 0), (OF != 0), (SP != 0), (VP != 0)>,    \
   "fa_fwd_mfma_" TN "_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)           \
       FA_CAT(FA_SFX_O_, OF) FA_CAT(FA_SFX_S_, SP) FA_CAT(FA_SFX_P_, VP)}
#define FA_V16_CVO(T, TN, DT, D, SP, VP)                                          \
  FA_V16(T, TN, DT, D, 0, 0, 0, SP, VP), FA_V16(T, TN, DT, D, 0, 0, 1, SP, VP),    \
  FA_V16(T, TN, DT, D, 0, 1, 0, SP, VP), FA_V16(T, TN, DT, D, 0, 1, 1, SP, VP),    \
  FA_V16(T, TN, DT, D, 1, 0, 0, SP, VP), FA_V16(T, TN, DT, D, 1, 0, 1, SP, VP),    \
  FA_V16(T, TN, DT, D, 1, 1, 0, SP, VP), FA_V16(T, TN, DT, D, 1, 1, 1, SP, VP)
#define FA_MFMA_TABLE(FN, T, TN, DT, D)                                           \
  namespace fa {                                                                  \
  const Variant* FN(int* n) {                                                     \
    static const Variant table[] = {                                              \
        FA_V16_CVO(T, TN, DT, D, 0, 0), FA_V16_CVO(T, TN, DT, D, 1, 0),            \
        FA_V16_CVO(T, TN, DT, D, 0, 1), FA_V16_CVO(T, TN, DT, D, 1, 1)};           \
    *n = (int)(sizeof(table) / sizeof(table[0]));                                 \
    return table;                                                                 \
  }                                                                               \
  }

#endif  // FA_FWD_MFMA_H
