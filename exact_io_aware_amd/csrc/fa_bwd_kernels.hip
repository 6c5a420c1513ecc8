// Exact attention backward for gfx950 (MI355X): dQ, dK, dV of sum(O * dO).
//
// What is computed (the derivative of the forward map, per head; the
// Kotaemon page "Kotaemon FlashAttention应用：加快注意力计算" describes the
// method as tiling plus recomputation, paragraph after the formula): with
// S = scale * Q K^T (masked), P = softmax(S) = exp(S - L) using the forward's
// per-row logsumexp L, and D_r = sum_j dO_rj O_rj,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// P is recomputed block by block from the saved L, so no N x N matrix is
// ever stored; grouped-query K/V gradients sum over the group's query heads.
//
// gfx950 mapping (our design):
//  * fa_bwd_delta: D_r, D/8 lanes per row (8 columns each).
//  * fa_bwd_dkdv: a workgroup of 8 waves owns 256 keys of one K/V head
//    (each wave 32 keys: its K rows in registers, its V rows in LDS, both
//    read as MFMA B operands) and streams 64-row query tiles (Q and dO,
//    row-major) of every query head of the group.  Per 32-row block it forms
//    S = Q K^T and dP = dO V^T (Q, dO read by rows), P and dS, then
//    dV^T += dO^T P and dK^T += Q^T dS (dO, Q read transposed).  S's
//    accumulator puts one key per lane column, which is exactly the
//    B-operand layout of P and dS for the gradient products, and the
//    transposing LDS reads deliver the query rows in that accumulator's
//    order.  No atomics.
//  * fa_bwd_dq: the forward kernel's structure: a wave owns 32 query rows
//    (Q and dO in registers), streams 64-key tiles of K and V (row-major),
//    forms S^T = K Q^T and dP^T = V dO^T with one query per lane column, and
//    accumulates dQ^T += K^T dS^T, K^T read from the same K tile.
//  * Every tile is row-major in LDS with the rm_swz layout, read by rows or
//    transposed (gfx950's ds_read_b64_tr_b16), so no transposed copy of any
//    tensor is made.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"
#include "fa_poison.h"

namespace fa {
namespace {

struct BwdParams {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;          // [B][Hq][N], natural log
  float* delta;              // [B][Hq][N], rowsum(dO * O)
  float* lse2;               // [B][Hq][N], lse * log2(e)
  void* dq; void* dk; void* dv;
  const int* cu_seqlens;
  int B, N, Hq, Hkv, G;
  int hp, rows_per_wg, n_rblocks, n_hgroups, xcd_remap;   // dq grid (as the forward)
  int rb_major, n_units;                         // dq order (as the forward)
  int kv_blocks;                                 // dV, dK: 256-key blocks per sequence
  float scale, scale_log2;
  long long q_bs, q_hs, q_rs;     // q, o, dO, dQ element strides
  long long kv_bs, kv_hs, kv_rs;  // k, v, dK, dV element strides
};

// ---------------------------------------------------------------------------
// D_r = sum_j dO_rj * O_rj (fp32), and L_r * log2(e) (the exponent offset
// of the base-2 exponentials).  D/8 lanes per row, 8 columns each: one
// 16-byte load of dO and one or two of O per lane.  HBM-bound (O and dO
// are read once), so the loads are non-temporal, the cache policy that
// streams fastest.
template <typename T, typename OT, int D, bool VARLEN>
__global__ __launch_bounds__(256) void fa_bwd_delta(BwdParams p) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPB = 256 / LPR;             // rows per workgroup
  const int row_id = blockIdx.x * RPB + (int)threadIdx.x / LPR;    // (b, h, r)
  const int sub = threadIdx.x % LPR;
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
  const long long off = (VARLEN ? (long long)(seq0 + r) * p.q_rs
                                : (long long)b * p.q_bs + (long long)r * p.q_rs) +
                        (long long)h * p.q_hs + 8 * sub;
  using vec8 = typename Ops<T>::vec8;
  const vec8 dv = __builtin_bit_cast(vec8, __builtin_nontemporal_load((const u32x4*)((const T*)p.dout + off)));
  float acc = 0.0f;
  if constexpr (std::is_same<OT, float>::value) {
    const f32x4* op = (const f32x4*)((const float*)p.o + off);
    const f32x4 o0 = __builtin_nontemporal_load(op), o1 = __builtin_nontemporal_load(op + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += (float)dv[j] * o0[j] + (float)dv[j + 4] * o1[j];
  } else {
    const vec8 ov = __builtin_bit_cast(vec8, __builtin_nontemporal_load((const u32x4*)((const T*)p.o + off)));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (float)dv[j] * (float)ov[j];
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (sub == 0) {
    const long long li = ((long long)b * p.Hq + h) * p.N + r;
    p.delta[li] = acc;
    p.lse2[li] = p.lse[li] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dV and dK in one pass.  One workgroup: 8 waves x 32 keys of K/V head g of
// sequence b; per 32-row query block: S = Q K^T, P, dP = dO V^T, dS,
// dV^T += dO^T P, dK^T += Q^T dS (tiles Q, dO; L, D).  With K rows, two
// score blocks and two 32 x d accumulators in registers there is no room
// for V as well, so each wave keeps its 32 V rows in LDS (rm_swz layout).
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32>
__global__ __launch_bounds__(512, 1) void fa_bwd_dkdv(BwdParams p) {
  using vec8 = typename Ops<T>::vec8;
  constexpr int NW = 8, NT = 512;
  constexpr int BR = 64;                     // query rows per tile (two 32-row blocks)
  constexpr int DB = D / 32, DC = D / 16, CPR = D / 8, RB = D * 2;
  constexpr int TILE_BYTES = BR * RB;
  constexpr int HALF = 32 * RB;
  constexpr int LOADS = BR * CPR / NT;       // 16-byte loads per thread per tile
  static_assert(LOADS >= 1 && BR * CPR == LOADS * NT, "tile fill");

  // Per buffer: Q and dO (row-major, rm_swz), L and D of the 64 rows.
  __shared__ __attribute__((aligned(16))) char q_l0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char q_l1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char do_l0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char do_l1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float ld_l0[2 * BR];   // L * log2(e), then D
  __shared__ __attribute__((aligned(16))) float ld_l1[2 * BR];
  // Each wave's 32 V rows.
  __shared__ __attribute__((aligned(16))) char v_own[NW * 32 * RB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(q_l0, TILE_BYTES, tid, NT);
    poison_lds(q_l1, TILE_BYTES, tid, NT);
    poison_lds(do_l0, TILE_BYTES, tid, NT);
    poison_lds(do_l1, TILE_BYTES, tid, NT);
    poison_lds(ld_l0, sizeof(ld_l0), tid, NT);
    poison_lds(ld_l1, sizeof(ld_l1), tid, NT);
    poison_lds(v_own, sizeof(v_own), tid, NT);
    __syncthreads();
  }

  // Key-block-major order: every (sequence, K/V head) takes its first key
  // block before any takes its second, so with the causal mask (early keys
  // are seen by the most queries) the longest workgroups start first.
  const int nbg = p.B * p.Hkv;
  const int kblk = blockIdx.x / nbg;
  const int bg = blockIdx.x - kblk * nbg;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  int seq0 = 0, len = p.N;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
  }
  const int kwg = kblk * (NW * 32);
  if (kwg >= len) return;                    // uniform
  const int kw0 = kwg + wave * 32;           // this wave's first key
  const bool wave_live = kw0 < len;          // wave-uniform
  const int key = kw0 + l32;                 // the key of this lane's S column

  const long long kvbase = (VARLEN ? (long long)seq0 * p.kv_rs : (long long)b * p.kv_bs) +
                           (long long)g * p.kv_hs;
  // Own K and V rows as B operands: lane (l32, hf) holds row key, columns
  // 16*dc + 8*hf .. +7 (V only until it is stored to LDS).
  vec8 kf[DC], vf[DC];
  {
    const int krows = __builtin_amdgcn_readfirstlane(max(0, min(32, len - kw0)));
    const long long at = kvbase + (long long)min(kw0, len) * p.kv_rs;
    const uint32_t bytes = (uint32_t)krows * (uint32_t)p.kv_rs * 2;
    const rsrc_t rk = make_rsrc((const T*)p.k + at, bytes);
    const uint32_t ko = (uint32_t)(l32 * p.kv_rs + hf * 8) * 2;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      kf[dc] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + dc * 32, 0, 0));
    const rsrc_t rv = make_rsrc((const T*)p.v + at, bytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      vf[dc] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(rv, ko + dc * 32, 0, 0));
  }

  // Tile fill offsets (row-major, rm_swz).
  uint32_t roff[LOADS];
  const uint32_t q_rs_bytes = (uint32_t)p.q_rs * 2;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pch = tid + NT * i;
    const int r = pch / CPR, pc = pch % CPR;
    roff[i] = r * q_rs_bytes + ((pc ^ rm_swz<D>(r)) << 4);
  }
  // Operand read addresses: by rows (query l32 of a 32-row block, 16-byte
  // chunk 2 dc + hf) and transposed (column block db).  The chunk index's dc
  // (db) bits lie above the bits the lane's own terms set, so the address
  // of chunk dc is raddr0 ^ 32 dc and that of column block db is
  // tbase0 ^ 64 db: two registers instead of DC + DB.
  const int raddr0 = l32 * RB + ((hf ^ rm_swz<D>(l32)) << 4);
  const int tbase0 = tr_base<D>(lane, 0);
  // The wave's V rows go to its LDS slot, row l32 chunk 2 dc + hf where a
  // row read of a tile finds it; only this wave reads them, after the
  // loop's first barrier.
  char* const vw = v_own + wave * 32 * RB;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) *(vec8*)(vw + (raddr0 ^ (32 * dc))) = vf[dc];

  // Iterations: (query head hh of the group, 64-row query tile t).
  const int t_first = CAUSAL ? kwg / BR : 0;
  const int nt = (len + BR - 1) / BR - t_first;   // query tiles per head
  const int n_it = p.G * nt;

  auto tile_load = [&](int hh, int t, char* ql, char* dol, float* ldl)
      __attribute__((always_inline)) {
    const int h = g * p.G + hh;
    const int qb = t * BR;
    const long long qbase = (VARLEN ? (long long)seq0 * p.q_rs : (long long)b * p.q_bs) +
                            (long long)h * p.q_hs;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(len - qb, BR)));
    const uint32_t rbytes = (uint32_t)rows * q_rs_bytes;
    const long long at = qbase + (long long)min(qb, len) * p.q_rs;
    const rsrc_t rq = make_rsrc((const T*)p.q + at, rbytes);
    const rsrc_t rdo = make_rsrc((const T*)p.dout + at, rbytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int o = (NT * i + 64 * wave) * 16;
      lds_load16(rq, ql + o, roff[i]);
      lds_load16(rdo, dol + o, roff[i]);
    }
    // L and D of the 64 rows (128 floats) from wave 0: lanes 0-15 fetch L
    // into ldl[0, 64), lanes 16-31 D into ldl[64, 128) (the LDS-direct
    // destination of lane L is base + 16 * L).
    if (wave == 0) {
      const long long lrow = ((long long)b * p.Hq + h) * p.N + qb;
      const rsrc_t rl = make_rsrc(p.lse2 + lrow, (uint32_t)rows * 4);
      if (lane < 16) {
        lds_load16(rl, (char*)ldl, lane * 16);
      } else if (lane < 32) {
        const rsrc_t rd = make_rsrc(p.delta + lrow, (uint32_t)rows * 4);
        lds_load16(rd, (char*)ldl, (lane - 16) * 16);
      }
    }
  };

  // dK^T and dV^T: column block db holds d rows 32 db .. 32 db + 31.
  f32x16 acc_k[DB], acc_v[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc_k[db] = f32x16{};
    acc_v[db] = f32x16{};
  }
  const float sl2 = p.scale_log2;

  // One 32-row query block (half hb of the tile in the given buffers).
  auto block = [&](int t, int hb, const char* ql, const char* dol, const float* ldl)
      __attribute__((always_inline)) {
    const int qr0 = t * BR + 32 * hb;          // first query row of the block
    // A block whose rows all precede this wave's keys (causal), or a wave
    // with no keys, adds nothing.
    if (!wave_live || (CAUSAL && qr0 + 31 < kw0)) return;
    __builtin_amdgcn_sched_barrier(0);
    // Per-block copies of the address bases, opaque to the compiler, so the
    // XOR-derived addresses are formed here and not kept across the loop.
    int ra = raddr0, tb = tbase0;
    asm volatile("" : "+v"(ra), "+v"(tb));
    // S = Q K^T and dP = dO V^T: element e of lane (key, hf) is query row
    // qr0 + 8*(e/4) + 4*hf + e%4.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const vec8 a = *(const vec8*)(ql + hb * HALF + (ra ^ (32 * dc)));
      s = Ops<T>::mfma(a, kf[dc], s);
    }
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const vec8 a = *(const vec8*)(dol + hb * HALF + (ra ^ (32 * dc)));
      const vec8 bv = *(const vec8*)(vw + (ra ^ (32 * dc)));
      dp = Ops<T>::mfma(a, bv, dp);
    }
    // Operand reads two MFMAs ahead of their use (the dP MFMAs read two
    // operands each).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * DC - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    // P and dS, packed to the input type (pkp, pkd); the masks are tested
    // only in blocks that cross the diagonal or an end of the sequence.
    uint32_t pkp[8], pkd[8];
    auto form = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int rl = 32 * hb + 8 * g4 + 4 * hf;   // row within the tile
        const f32x4 L4 = *(const f32x4*)(ldl + rl);
        const f32x4 D4 = *(const f32x4*)(ldl + BR + rl);
        float pe[4], pp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * g4 + j;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sl2, -L4[j]));
          if (decltype(masked)::value) {
            const int qr = qr0 + 8 * g4 + 4 * hf + j;
            if (qr >= len || key >= len || (CAUSAL && key > qr)) pv = 0.0f;
          }
          pp[j] = pv;
          pe[j] = pv * (dp[e] - D4[j]);
        }
        pkp[2 * g4] = Ops<T>::pack(pp[0], pp[1]);
        pkp[2 * g4 + 1] = Ops<T>::pack(pp[2], pp[3]);
        pkd[2 * g4] = Ops<T>::pack(pe[0], pe[1]);
        pkd[2 * g4 + 1] = Ops<T>::pack(pe[2], pe[3]);
      }
    };
    if (qr0 + 31 >= len || kw0 + 31 >= len || (CAUSAL && kw0 + 31 > qr0))
      form(BoolTag<true>{});
    else
      form(BoolTag<false>{});
    __builtin_amdgcn_sched_barrier(0);
    // dK^T += Q^T dS and dV^T += dO^T P over the block's two 16-row chunks
    // (Q and dO read transposed from their tiles).
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 db4 = {pkd[4 * kc], pkd[4 * kc + 1], pkd[4 * kc + 2], pkd[4 * kc + 3]};
      const u32x4 pb4 = {pkp[4 * kc], pkp[4 * kc + 1], pkp[4 * kc + 2], pkp[4 * kc + 3]};
      const vec8 dsf = __builtin_bit_cast(vec8, db4), pf = __builtin_bit_cast(vec8, pb4);
      const int r0 = 32 * hb + 16 * kc;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int t0 = tb ^ (64 * db), t1 = tb ^ (64 * db + 32);
        const vec8 qa = lds_read_tr<vec8>(ql + t0 + r0 * RB, ql + t1 + (r0 + 8) * RB);
        acc_k[db] = Ops<T>::mfma(qa, dsf, acc_k[db]);
        const vec8 da = lds_read_tr<vec8>(dol + t0 + r0 * RB, dol + t1 + (r0 + 8) * RB);
        acc_v[db] = Ops<T>::mfma(da, pf, acc_v[db]);
      }
    }
    // Gradient MFMAs, two transposing reads each.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Iteration it is (query head hh, tile t); the pair advances without a
  // division.
  auto next = [&](int& hh, int& t) __attribute__((always_inline)) {
    if (++t == t_first + nt) {
      t = t_first;
      ++hh;
    }
  };
  int h0 = 0, t0 = t_first, h1 = 0, t1 = t_first;
  next(h1, t1);
  if (n_it > 0) tile_load(h0, t0, q_l0, do_l0, ld_l0);
  for (int it = 0; it < n_it; it += 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (it + 1 < n_it) tile_load(h1, t1, q_l1, do_l1, ld_l1);
    block(t0, 0, q_l0, do_l0, ld_l0);
    block(t0, 1, q_l0, do_l0, ld_l0);
    if (it + 1 >= n_it) break;
    h0 = h1;
    t0 = t1;
    next(h0, t0);                              // iteration it + 2
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (it + 2 < n_it) tile_load(h0, t0, q_l0, do_l0, ld_l0);
    block(t1, 0, q_l1, do_l1, ld_l1);
    block(t1, 1, q_l1, do_l1, ld_l1);
    h1 = h0;
    t1 = t0;
    next(h1, t1);                              // iteration it + 3
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // dK = scale * (dK^T)^T and dV: lane = key, rows 32*db + 8*g4 + 4*hf + 0..3.
  auto store = [&](const f32x16 (&a)[DB], void* out, float f) __attribute__((always_inline)) {
    const long long row = kvbase + (long long)key * p.kv_rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        const float a0 = a[db][4 * g4] * f, a1 = a[db][4 * g4 + 1] * f;
        const float a2 = a[db][4 * g4 + 2] * f, a3 = a[db][4 * g4 + 3] * f;
        if (OUT_F32)
          *(f32x4*)((float*)out + row + d0) = f32x4{a0, a1, a2, a3};
        else
          *(u32x2*)((T*)out + row + d0) = u32x2{Ops<T>::pack(a0, a1), Ops<T>::pack(a2, a3)};
      }
  };
  if (key < len) {
    store(acc_k, p.dk, p.scale);
    store(acc_v, p.dv, 1.0f);
  }
}

// ---------------------------------------------------------------------------
// dQ.  The forward kernel's layout: 8 waves, each 32 query rows of one head
// (up to 4 heads of a K/V group per workgroup), 64-key tiles of K and V
// double-buffered in LDS; K^T is the K tile read transposed.
template <typename T, int D, bool CAUSAL, bool VARLEN, bool OUT_F32>
__global__ __launch_bounds__(64 * waves_per_wg(FA_BF16, D, CAUSAL), 2) void fa_bwd_dq(BwdParams p) {
  using vec8 = typename Ops<T>::vec8;
  // 8 waves (4 at d = 64 under the causal mask: the forward kernel's
  // choice, for the same reasons).
  constexpr int NT = 64 * waves_per_wg(FA_BF16, D, CAUSAL);
  constexpr int BC = 64;
  constexpr int DB = D / 32, DC = D / 16, CPR = D / 8, RB = D * 2;
  constexpr int TILE_BYTES = BC * RB;
  constexpr int HALF = 32 * RB;
  constexpr int LOADS = BC * CPR / NT;

  __shared__ __attribute__((aligned(16))) char k_l0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_l1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_l0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_l1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  if constexpr (kPoisonLds) {                // test build only
    poison_lds(k_l0, TILE_BYTES, tid, NT);
    poison_lds(k_l1, TILE_BYTES, tid, NT);
    poison_lds(v_l0, TILE_BYTES, tid, NT);
    poison_lds(v_l1, TILE_BYTES, tid, NT);
    __syncthreads();
  }

  // Workgroups are dealt round-robin over the 8 XCDs (workgroup j on XCD
  // j % 8).  With xcd_remap, XCD x takes the units u with u % 8 == x, each
  // unit's row blocks consecutively (as the forward kernel): a unit's K/V
  // stays in one XCD's L2, and every XCD gets the same mix of long and
  // short causal row blocks.  With rb_major, row-block slot s of every unit
  // comes before slot s + 1 of any (longest row blocks of all units first).
  const int idx = p.xcd_remap ? blockIdx.x >> 3 : blockIdx.x;
  const int nu = p.xcd_remap ? p.n_units >> 3 : p.n_units;
  int k, rb;
  if (p.rb_major) {
    rb = idx / nu;
    k = idx - rb * nu;
  } else {
    k = idx / p.n_rblocks;
    rb = idx - k * p.n_rblocks;
  }
  const int unit = p.xcd_remap ? 8 * k + (blockIdx.x & 7) : k;
  const int b = unit / p.n_hgroups;
  const int hgrp = unit - b * p.n_hgroups;
  const int h = hgrp * p.hp + (wave % p.hp);
  const int kvh = (hgrp * p.hp) / p.G;
  int seq0 = 0, len = p.N;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    len = p.cu_seqlens[b + 1] - seq0;
  }
  // Longest row blocks first: the sequence's last ones (slot s is row
  // block nrb - 1 - s).
  if (CAUSAL) rb = (VARLEN ? (len + p.rows_per_wg - 1) / p.rows_per_wg : p.n_rblocks) - 1 - rb;
  const int wg_row0 = rb * p.rows_per_wg;
  if (rb < 0 || wg_row0 >= len) return;
  const int row0 = wg_row0 + (wave / p.hp) * 32;
  const int kv_end = CAUSAL ? min(wg_row0 + p.rows_per_wg, len) : len;
  const bool active = row0 < len;
  const int qrow = row0 + l32;

  const long long qbase = (VARLEN ? (long long)seq0 * p.q_rs : (long long)b * p.q_bs) +
                          (long long)h * p.q_hs;
  const long long kvbase = (VARLEN ? (long long)seq0 * p.kv_rs : (long long)b * p.kv_bs) +
                           (long long)kvh * p.kv_hs;
  const uint32_t kv_rs_bytes = (uint32_t)p.kv_rs * 2;

  // Q and dO rows as B operands; this lane's L (log2 units) and D.
  vec8 qf[DC], df[DC];
  float l2 = __builtin_inff(), dl = 0.0f;
  {
    const int qrows = __builtin_amdgcn_readfirstlane(active ? min(32, len - row0) : 0);
    const uint32_t bytes = (uint32_t)qrows * (uint32_t)p.q_rs * 2;
    const rsrc_t rq = make_rsrc((const T*)p.q + qbase + (long long)(active ? row0 : 0) * p.q_rs, bytes);
    const rsrc_t rd = make_rsrc((const T*)p.dout + qbase + (long long)(active ? row0 : 0) * p.q_rs,
                                bytes);
    const uint32_t qo = (uint32_t)(l32 * p.q_rs + hf * 8) * 2;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      qf[dc] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(rq, qo + dc * 32, 0, 0));
      df[dc] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(rd, qo + dc * 32, 0, 0));
    }
    if (active && qrow < len) {
      const long long li = ((long long)b * p.Hq + h) * p.N + qrow;
      l2 = p.lse[li] * kLog2e;
      dl = p.delta[li];
    }
  }

  auto tile_load = [&](int t, char* kl, char* vl) __attribute__((always_inline)) {
    // The per-lane fill offsets are recomputed at each tile (a few integer
    // instructions) rather than kept in registers across the loop, where
    // they would be spilled.
    int tid_t = tid;
    asm volatile("" : "+v"(tid_t));
    uint32_t koff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int pch = tid_t + NT * i;
      const int r = pch / CPR, pc = pch % CPR;
      koff[i] = r * kv_rs_bytes + ((pc ^ rm_swz<D>(r)) << 4);
    }
    const int kb = t * BC;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(len - kb, BC)));
    const long long at = (long long)min(kb, len) * p.kv_rs;
    const rsrc_t rk = make_rsrc((const T*)p.k + kvbase + at, (uint32_t)rows * kv_rs_bytes);
    const rsrc_t rv = make_rsrc((const T*)p.v + kvbase + at, (uint32_t)rows * kv_rs_bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int o = (NT * i + 64 * wave) * 16;
      lds_load16(rk, kl + o, koff[i]);
      lds_load16(rv, vl + o, koff[i]);
    }
  };
  // Operand read addresses: K and V by rows (key l32 of a 32-key block,
  // 16-byte chunk 2 dc + hf), K transposed (column block db).
  int kaddr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) kaddr[dc] = l32 * RB + (((2 * dc + hf) ^ rm_swz<D>(l32)) << 4);
  int tbase[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) tbase[db] = tr_base<D>(lane, db);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  const float sl2 = p.scale_log2;

  auto block = [&](int t, int hb, const char* kl, const char* vl)
      __attribute__((always_inline)) {
    const int kb = t * BC + 32 * hb;
    // d = 64: a wave without rows, or (causal) a block wholly past the
    // wave's last row, adds nothing (P = 0 there) and is skipped; the loads
    // and barriers are shared.  (At d = 128 the skip changed the register
    // allocation and measured 0.5 % slower on gqa_bf16.)
    if constexpr (D == 64) {
      if (!active || (CAUSAL && kb > row0 + 31)) return;
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const vec8 a = *(const vec8*)(kl + hb * HALF + kaddr[dc]);
      s = Ops<T>::mfma(a, qf[dc], s);
    }
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const vec8 a = *(const vec8*)(vl + hb * HALF + kaddr[dc]);
      dp = Ops<T>::mfma(a, df[dc], dp);
    }
    // Operand reads two MFMAs ahead of their use, one per MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * DC - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    // Element e of lane (query, hf) is key kb + 8*(e/4) + 4*hf + e%4.  Only
    // a block that crosses the diagonal or the end of the sequence is masked
    // (scores set to -inf, so P = 0); rows past the end have l2 = +inf.
    if ((CAUSAL && kb + 31 > row0) || kb + 32 > len) {
      const int lim = (CAUSAL ? min(len, qrow + 1) : len) - kb - 4 * hf;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) >= lim) s[e] = -__builtin_inff();
    }
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float ds[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + j], sl2, -l2));
        ds[j] = pv * (dp[e + j] - dl);
      }
      pk[e >> 1] = Ops<T>::pack(ds[0], ds[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T (K read transposed from its tile).
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 sb = {pk[4 * kc], pk[4 * kc + 1], pk[4 * kc + 2], pk[4 * kc + 3]};
      const vec8 sf = __builtin_bit_cast(vec8, sb);
      const int r0 = 32 * hb + 16 * kc;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const vec8 a = lds_read_tr<vec8>(kl + tbase[db] + r0 * RB,
                                         kl + (tbase[db] ^ 32) + (r0 + 8) * RB);
        acc[db] = Ops<T>::mfma(a, sf, acc[db]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int ntl = (kv_end + BC - 1) / BC;
  tile_load(0, k_l0, v_l0);
  for (int t = 0; t < ntl; t += 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (t + 1 < ntl) tile_load(t + 1, k_l1, v_l1);
    block(t, 0, k_l0, v_l0);
    block(t, 1, k_l0, v_l0);
    if (t + 1 >= ntl) break;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (t + 2 < ntl) tile_load(t + 2, k_l0, v_l0);
    block(t + 1, 0, k_l1, v_l1);
    block(t + 1, 1, k_l1, v_l1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  if (!active || qrow >= len) return;
  const long long orow = qbase + (long long)qrow * p.q_rs;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * hf;
      const float a0 = acc[db][4 * g4] * p.scale, a1 = acc[db][4 * g4 + 1] * p.scale;
      const float a2 = acc[db][4 * g4 + 2] * p.scale, a3 = acc[db][4 * g4 + 3] * p.scale;
      if (OUT_F32) {
        *(f32x4*)((float*)p.dq + orow + d0) = f32x4{a0, a1, a2, a3};
      } else {
        *(u32x2*)((T*)p.dq + orow + d0) = u32x2{Ops<T>::pack(a0, a1), Ops<T>::pack(a2, a3)};
      }
    }
}

// ---------------------------------------------------------------------------
// Dispatch.
typedef void (*BwdFn)(BwdParams);

struct BwdVariant {
  int in_dtype, d, causal, varlen, grad_f32;
  BwdFn dkdv, dq;
};

#define FA_BV(T, DT, D, C, VL, OF)                                                     \
  {DT, D, C, VL, OF, fa_bwd_dkdv<T, D, (C != 0), (VL != 0), (OF != 0)>,                  \
   fa_bwd_dq<T, D, (C != 0), (VL != 0), (OF != 0)>}
#define FA_BV_ALL(T, DT, D)                                                             \
  FA_BV(T, DT, D, 0, 0, 0), FA_BV(T, DT, D, 0, 0, 1), FA_BV(T, DT, D, 0, 1, 0),           \
  FA_BV(T, DT, D, 0, 1, 1), FA_BV(T, DT, D, 1, 0, 0), FA_BV(T, DT, D, 1, 0, 1),           \
  FA_BV(T, DT, D, 1, 1, 0), FA_BV(T, DT, D, 1, 1, 1)

const BwdVariant kBwdVariants[] = {
    FA_BV_ALL(__bf16, FA_BF16, 64), FA_BV_ALL(__bf16, FA_BF16, 128),
    FA_BV_ALL(_Float16, FA_F16, 64), FA_BV_ALL(_Float16, FA_F16, 128),
};

struct DeltaVariant {
  int in_dtype, o_f32, d, varlen;
  BwdFn fn;
};
#define FA_DV(T, DT, D)                                                                 \
  {DT, 0, D, 0, fa_bwd_delta<T, T, D, false>}, {DT, 0, D, 1, fa_bwd_delta<T, T, D, true>}, \
  {DT, 1, D, 0, fa_bwd_delta<T, float, D, false>},                                       \
  {DT, 1, D, 1, fa_bwd_delta<T, float, D, true>}
const DeltaVariant kDeltaVariants[] = {
    FA_DV(__bf16, FA_BF16, 64), FA_DV(__bf16, FA_BF16, 128),
    FA_DV(_Float16, FA_F16, 64), FA_DV(_Float16, FA_F16, 128),
};

}  // namespace

// Workspace layout of the backward pass: D and L * log2(e), fp32 rows
// [B][Hq][N], each padded to 256 B.
struct BwdLayout {
  uint64_t delta, lse2, total;
};
static BwdLayout bwd_layout(int B, int Hq, int Hkv, int N, int d) {
  (void)Hkv;
  (void)d;
  BwdLayout l;
  const uint64_t rows = (uint64_t)B * Hq * N;
  l.delta = 0;
  l.lse2 = (rows * 4 + 255) & ~255ull;
  l.total = 2 * l.lse2;
  return l;
}

int launch_bwd(const BwdArgs& a, void* stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  const BwdVariant* var = nullptr;
  for (const BwdVariant& v : kBwdVariants)
    if (v.in_dtype == a.in_dtype && v.d == a.d && v.causal == a.causal &&
        v.varlen == (int)varlen && v.grad_f32 == (a.grad_dtype == FA_F32))
      var = &v;
  const DeltaVariant* dv = nullptr;
  for (const DeltaVariant& v : kDeltaVariants)
    if (v.in_dtype == a.in_dtype && v.o_f32 == (a.o_dtype == FA_F32) && v.d == a.d &&
        v.varlen == (int)varlen)
      dv = &v;
  if (!var || !dv) return FA_ERR_DTYPE;
  const BwdLayout lay = bwd_layout(a.B, a.Hq, a.Hkv, a.N, a.d);
  char* ws = (char*)a.workspace;

  BwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.dout = a.dout; p.lse = a.lse;
  p.delta = (float*)(ws + lay.delta);
  p.lse2 = (float*)(ws + lay.lse2);
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv;
  p.cu_seqlens = a.cu_seqlens;
  p.B = a.B; p.N = a.N; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv;
  const int dq_threads = 64 * waves_per_wg(a.in_dtype, a.d, a.causal);  // as the dQ kernel
  const Plan plan = make_plan_nw(a.B, a.Hq, a.Hkv, a.N, a.in_dtype, dq_threads / 64);
  p.hp = plan.hp; p.rows_per_wg = plan.rows_per_wg; p.n_rblocks = plan.n_rblocks;
  p.n_hgroups = plan.n_hgroups;
  p.xcd_remap = ((uint64_t)a.B * plan.n_hgroups) % 8 == 0;
  p.n_units = a.B * plan.n_hgroups;
  // Row-block-major only for a launch a few rounds deep whose K/V all fits
  // in half of the last-level cache (the forward's rule).
  p.rb_major = 0;
  if (a.causal && 4LL * a.B * a.Hkv * a.N * a.d <= (128LL << 20)) {
    int dev = -1, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)var->dq, dq_threads, 0) ==
            hipSuccess &&
        cus > 0 && per_cu > 0)
      p.rb_major = plan.total_wg <= 4ull * (uint64_t)cus * (uint64_t)per_cu;
  }
  if (const int fo = forced_order(); fo >= 0) {     // a test of order independence
    p.xcd_remap = (fo & 1) && p.n_units % 8 == 0;
    p.rb_major = (fo & 2) ? 1 : 0;
  }
  p.kv_blocks = (a.N + 255) / 256;
  p.scale = a.scale; p.scale_log2 = a.scale * kLog2e;
  const long long d = a.d;
  if (varlen) {
    p.q_bs = 0; p.q_hs = d; p.q_rs = (long long)a.Hq * d;
    p.kv_bs = 0; p.kv_hs = d; p.kv_rs = (long long)a.Hkv * d;
  } else {
    p.q_rs = d; p.q_hs = (long long)a.N * d; p.q_bs = (long long)a.Hq * a.N * d;
    p.kv_rs = d; p.kv_hs = (long long)a.N * d; p.kv_bs = (long long)a.Hkv * a.N * d;
  }
  hipStream_t s = (hipStream_t)stream;
  void* args[] = {&p};
  const uint64_t rows = (uint64_t)a.B * a.Hq * a.N;
  const uint64_t rpb = 256 / (a.d / 8);      // fa_bwd_delta: rows per workgroup
  if (hipLaunchKernel((const void*)dv->fn, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256),
                      args, 0, s) != hipSuccess)
    return FA_ERR_LAUNCH;
  const unsigned g1 = (unsigned)((uint64_t)a.B * a.Hkv * p.kv_blocks);
  if (hipLaunchKernel((const void*)var->dkdv, dim3(g1), dim3(512), args, 0, s) != hipSuccess)
    return FA_ERR_LAUNCH;
  if (hipLaunchKernel((const void*)var->dq, dim3((unsigned)plan.total_wg), dim3(dq_threads), args, 0,
                      s) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace fa
