// Forward kernels other than the main 16-bit attention kernel (which lives
// in fa_fwd_mfma.h, instantiated per input type and head dimension), and the
// launch logic of every forward entry point:
//  * fa_vt_pack: V transposed into 64-key tiles (the decode cache's layout);
//  * fa_decode_mfma: few query rows per sequence against a long K/V cache;
//  * fa_merge_splits: the split-KV merge;
//  * fa_fwd_f32: fp32 inputs on fp32 MFMA;
//  * fa_check_seqlens_kernel: the debug-mode check of packed offsets.
// What they compute is the attention of fa_fwd (the Kotaemon page,
// "Kotaemon FlashAttention应用：加快注意力计算", formula paragraph and
// method list; O together with the normaliser L, as the tiling sketch of the
// French HolySheep Flash Attention article returns).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_fwd_common.h"
#include "fa_internal.h"
#include "fa_poison.h"

namespace fa {
namespace {

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
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(vl, sizeof(vl), tid, blockDim.x);
    __syncthreads();
  }
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
// VPACK: V comes as packed V^T tiles (fa_vt_pack); otherwise V's rows are
// staged row-major and read transposed (ds_read_b64_tr_b16).
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32, bool VPACK>
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
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(slots, sizeof(slots), tid, blockDim.x);
    poison_lds(q_lds, sizeof(q_lds), tid, blockDim.x);
    poison_lds(m_s, sizeof(m_s), tid, blockDim.x);
    poison_lds(l_s, sizeof(l_s), tid, blockDim.x);
    __syncthreads();
  }

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
  const char* vp = (const char*)((const T*)p.v + kvbase);
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
      // scale < 0: Q negated; scale = 0: Q zero (see FwdParams::q_mode).
      if (p.q_mode == 1) v = u32x4{v[0] ^ 0x80008000u, v[1] ^ 0x80008000u, v[2] ^ 0x80008000u,
                                   v[3] ^ 0x80008000u};
      if (p.q_mode == 2) v = u32x4{0u, 0u, 0u, 0u};
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
  // pc), then the V^T tile (row vr = position / 8 of 128 B, chunk vc) or,
  // row-major, the 64 V rows as the K rows.
  // Rows past the sequence end, and tiles past the wave's last, read zeros
  // (bounded buffers); the loads are issued unconditionally so every path
  // keeps the same loads in flight.
  struct Stage { u32x4 x[LOADS]; };
  struct TileRes { rsrc_t rk, rv; };
  auto tile_res = [&](int j) __attribute__((always_inline)) -> TileRes {
    const int t = t0 + wave + NW * j;
    const int kb = 64 * t;
    const bool in = j < my_tiles;
    const int rows = __builtin_amdgcn_readfirstlane(in ? max(0, min(len_k - kb, 64)) : 0);
    TileRes r;
    r.rk = make_rsrc(kp + (long long)min(kb, len_k) * kv_rs_bytes, (uint32_t)rows * kv_rs_bytes);
    r.rv = VPACK ? make_rsrc(vtp + (long long)(in ? t : 0) * TILE_BYTES,
                             in ? (uint32_t)TILE_BYTES : 0u)
                 : make_rsrc(vp + (long long)min(kb, len_k) * kv_rs_bytes,
                             (uint32_t)rows * kv_rs_bytes);
    return r;
  };
  auto gload1 = [&](const TileRes& r, int i) __attribute__((always_inline)) -> u32x4 {
    const int q = 64 * i + lane;
    if (i < TILE_BYTES / 1024) {
      const int rr = q / CPR, pc = q % CPR;
      return __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rk, rr * kv_rs_bytes + 16 * pc, 0, kNT));
    } else if (VPACK) {
      return __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rv, 16 * (q - TILE_BYTES / 16), 0, kNT));
    } else {
      const int qv = q - TILE_BYTES / 16;
      const int rr = qv / CPR, pc = qv % CPR;
      return __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rv, rr * kv_rs_bytes + 16 * pc, 0, kNT));
    }
  };
  // ... and into the wave's LDS slot, swizzled for the operand reads: K
  // chunk pc of row r at position pc ^ k_swz(r) (rows of RB bytes); V^T
  // chunk vc of row vr at vc ^ vt_swz(vr) (rows of 128 bytes); row-major V
  // chunk pc of row r at pc ^ rm_swz(r) (rows of RB bytes).
  char* const my_slot = slots + wave * STAGE;
  auto swrite1 = [&](const u32x4& x, int i) __attribute__((always_inline)) {
    const int q = 64 * i + lane;
    if (i < TILE_BYTES / 1024) {
      const int r = q / CPR, pc = q % CPR;
      *(u32x4*)(my_slot + r * RB + ((pc ^ k_swz<D>(r)) << 4)) = x;
    } else if (VPACK) {
      const int qv = q - TILE_BYTES / 16;
      const int vr = qv >> 3, vc = qv & 7;
      *(u32x4*)(my_slot + TILE_BYTES + vr * 128 + ((vc ^ vt_swz(vr)) << 4)) = x;
    } else {
      const int qv = q - TILE_BYTES / 16;
      const int r = qv / CPR, pc = qv % CPR;
      *(u32x4*)(my_slot + TILE_BYTES + r * RB + ((pc ^ rm_swz<D>(r)) << 4)) = x;
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
  // Row-major V: transposing-read offsets of output block db (second half
  // of a 16-row chunk at vtr ^ 32, see fa_fwd_mfma).
  int vtr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) vtr[db] = TILE_BYTES + tr_base<D>(lane, db);

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
        vec8 vf;
        if constexpr (VPACK) {
          vf = *(const vec8*)(my_slot + db * 32 * 128 + (vaddr0 ^ (32 * (2 * h + kc))));
        } else {
          const int r0 = 32 * h + 16 * kc;
          vf = lds_read_tr<vec8>(my_slot + vtr[db] + r0 * RB,
                                 my_slot + (vtr[db] ^ 32) + (r0 + 8) * RB);
        }
        oacc[db] = Ops<T>::mfma(vf, pf, oacc[db]);
      }
    }
  };

  // Tile j + 1 loads into the registers while tile j, written to the slot,
  // is computed (its second half only when it holds keys before k_stop).
  // Each staged register is reloaded with tile j + 1 as soon as its part of
  // tile j is in the slot, so a wave keeps a whole tile's loads in flight.
  Stage st;
  {
    const TileRes r0 = tile_res(0);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) st.x[i] = gload1(r0, i);
  }
  for (int j = 0; j < my_tiles; ++j) {
    const TileRes rn = tile_res(j + 1);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      swrite1(st.x[i], i);
      st.x[i] = gload1(rn, i);
    }
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
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(ks, sizeof(ks), tid, blockDim.x);
    poison_lds(vs, sizeof(vs), tid, blockDim.x);
    __syncthreads();
  }

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
    // scale < 0: Q negated; scale = 0: Q zero (see FwdParams::q_mode).
    if (p.q_mode != 0) {
#pragma unroll
      for (int t = 0; t < DK; ++t) qf[t] = p.q_mode == 1 ? -qf[t] : 0.0f;
    }
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
// Debug check of packed offsets (FA_DEBUG=1): entry i of cu (i = 0 .. B)
// must satisfy seqlens_entry_ok (cu[0] = 0, non-decreasing, each length at
// most n_max).  One workgroup; the outcome (0 good, 1 bad) goes to *bad.
__global__ __launch_bounds__(256) void fa_check_seqlens_kernel(const int* cu, int B, int n_max,
                                                               int* bad) {
  int fail = 0;
  for (int i = threadIdx.x; i <= B; i += 256)
    fail |= seqlens_entry_ok(i, i > 0 ? cu[i - 1] : 0, cu[i], n_max) ? 0 : 1;
  fail = __syncthreads_or(fail);
  if (threadIdx.x == 0) *bad = fail != 0 ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Dispatch tables.
#define FA_SFX_C_0 ""
#define FA_SFX_C_1 "_causal"
#define FA_SFX_V_0 ""
#define FA_SFX_V_1 "_varlen"
#define FA_SFX_O_0 ""
#define FA_SFX_O_1 "_of32"
#define FA_SFX_P_0 ""
#define FA_SFX_P_1 "_vtpacked"
#define FA_CAT(a, b) a##b
#define FA_V32(D, C, VL)                                                           \
  {FA_F32, D, C, VL, FA_F32, 0, 0, fa_fwd_f32<D, (C != 0), (VL != 0)>,             \
   "fa_fwd_f32_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)}

const Variant kF32Variants[] = {
    FA_V32(64, 0, 0), FA_V32(64, 0, 1), FA_V32(64, 1, 0), FA_V32(64, 1, 1),
    FA_V32(128, 0, 0), FA_V32(128, 0, 1), FA_V32(128, 1, 0), FA_V32(128, 1, 1),
};

// Decode kernels (16-bit inputs, G * Nq <= 32).
struct DecodeVariant {
  int in_dtype, d, causal, varlen, out_dtype, vpack;
  KernelFn fn;
  const char* name;
};
#define FA_VD(T, TN, DT, D, C, VL, OF, VP)                                        \
  {DT, D, C, VL, (OF) ? FA_F32 : DT, VP,                                          \
   fa_decode_mfma<T, D, (C != 0), (VL != 0), (OF != 0), (VP != 0)>,               \
   "fa_decode_mfma_" TN "_d" #D FA_CAT(FA_SFX_C_, C) FA_CAT(FA_SFX_V_, VL)         \
       FA_CAT(FA_SFX_O_, OF) FA_CAT(FA_SFX_P_, VP)}
#define FA_VD_ALL(T, TN, DT, D, VP)                                               \
  FA_VD(T, TN, DT, D, 0, 0, 0, VP), FA_VD(T, TN, DT, D, 0, 0, 1, VP),              \
  FA_VD(T, TN, DT, D, 0, 1, 0, VP), FA_VD(T, TN, DT, D, 0, 1, 1, VP),              \
  FA_VD(T, TN, DT, D, 1, 0, 0, VP), FA_VD(T, TN, DT, D, 1, 0, 1, VP),              \
  FA_VD(T, TN, DT, D, 1, 1, 0, VP), FA_VD(T, TN, DT, D, 1, 1, 1, VP)
const DecodeVariant kDecodeVariants[] = {
    FA_VD_ALL(__bf16, "bf16", FA_BF16, 64, 0), FA_VD_ALL(__bf16, "bf16", FA_BF16, 128, 0),
    FA_VD_ALL(_Float16, "f16", FA_F16, 64, 0), FA_VD_ALL(_Float16, "f16", FA_F16, 128, 0),
    FA_VD_ALL(__bf16, "bf16", FA_BF16, 64, 1), FA_VD_ALL(__bf16, "bf16", FA_BF16, 128, 1),
    FA_VD_ALL(_Float16, "f16", FA_F16, 64, 1), FA_VD_ALL(_Float16, "f16", FA_F16, 128, 1),
};
const DecodeVariant* find_decode(int in_dtype, int d, int causal, int varlen, int out_dtype,
                                 int vpack) {
  for (const DecodeVariant& v : kDecodeVariants)
    if (v.in_dtype == in_dtype && v.d == d && v.causal == causal && v.varlen == varlen &&
        v.out_dtype == out_dtype && v.vpack == vpack)
      return &v;
  return nullptr;
}

const Variant* find_variant(int in_dtype, int d, int causal, int varlen, int out_dtype,
                            int sparse = 0, int vpack = 0) {
  auto match = [&](const Variant& v) {
    return v.in_dtype == in_dtype && v.d == d && v.causal == causal && v.varlen == varlen &&
           v.out_dtype == out_dtype && v.sparse == sparse && v.vpack == vpack;
  };
  if (in_dtype == FA_F32) {
    for (const Variant& v : kF32Variants)
      if (match(v)) return &v;
    return nullptr;
  }
  const Variant* (*tables[])(int*) = {mfma_variants_bf16_d64, mfma_variants_bf16_d128,
                                      mfma_variants_f16_d64, mfma_variants_f16_d128};
  for (auto get : tables) {
    int n = 0;
    const Variant* t = get(&n);
    for (int i = 0; i < n; ++i)
      if (match(t[i])) return &t[i];
  }
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
                           int Hkv, int Nq, int sparse, int vpack) {
  if (use_decode(in_dtype, Hq, Hkv, Nq, sparse != 0)) {
    const DecodeVariant* v =
        find_decode(in_dtype, d, causal != 0, varlen != 0, out_dtype, vpack != 0);
    return v ? v->name : nullptr;
  }
  const Variant* v = find_variant(in_dtype, d, causal != 0, varlen != 0, out_dtype,
                                  sparse != 0, in_dtype == FA_F32 ? 0 : vpack != 0);
  return v ? v->name : nullptr;
}

// The debug check's outcome, one per device.
__device__ int g_seqlens_bad;

// Fixed device memory for the split-KV partials of fa_fwd_kv_split_noalloc
// (callers that cannot allocate: graph capture, serving loops).  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_ptr[dev] =
        hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

int debug_check_seqlens(const int* cu, int B, int n_max, void* stream) {
  static std::mutex mu;                       // one outcome slot per device
  std::lock_guard<std::mutex> lock(mu);
  int* bad = nullptr;
  if (hipGetSymbolAddress((void**)&bad, HIP_SYMBOL(g_seqlens_bad)) != hipSuccess || !bad)
    return FA_ERR_LAUNCH;
  void* args[] = {(void*)&cu, (void*)&B, (void*)&n_max, (void*)&bad};
  if (hipLaunchKernel((const void*)fa_check_seqlens_kernel, dim3(1), dim3(256), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return FA_ERR_LAUNCH;
  int outcome = 1;
  if (hipMemcpyAsync(&outcome, bad, sizeof(int), hipMemcpyDeviceToHost, (hipStream_t)stream) !=
          hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return FA_ERR_LAUNCH;
  return outcome == 0 ? FA_OK : FA_ERR_SEQLENS;
}

int launch_fwd(const LaunchArgs& a, void* stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  const bool sparse = a.block_mask != nullptr;
  const bool vpack = a.vt != nullptr;
  if ((sparse || vpack) && a.in_dtype == FA_F32) return FA_ERR_DTYPE;
  const Variant* var = find_variant(a.in_dtype, a.d, a.causal, varlen, a.out_dtype, sparse, vpack);
  if (!var) return FA_ERR_DTYPE;
  const bool decode = use_decode(a.in_dtype, a.Hq, a.Hkv, a.N, sparse);
  const DecodeVariant* dvar =
      decode ? find_decode(a.in_dtype, a.d, a.causal, varlen, a.out_dtype, vpack) : nullptr;
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
  // scale < 0 and scale = 0 enter through Q (q_mode), the kernels keep a
  // positive scale.
  p.q_mode = a.scale < 0.0f ? 1 : a.scale == 0.0f ? 2 : 0;
  p.scale_log2 = (a.scale < 0.0f ? -a.scale : a.scale == 0.0f ? 1.0f : a.scale) * kLog2e;
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
  if (const int fo = forced_order(); fo >= 0) {     // a test of order independence
    p.xcd_remap = (fo & 1) && a.in_dtype != FA_F32 && n_splits == 1 && p.n_units % 8 == 0;
    p.rb_major = (fo & 2) ? 1 : 0;
  }
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
