// Device helpers shared by the forward and backward attention kernels
// (types, MFMA element traits, buffer resources, LDS-direct loads, LDS
// swizzles, the P.V fragment key order).  Included by the .hip sources only.
#ifndef FA_DEVICE_H
#define FA_DEVICE_H

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Largest partial row sum of P tolerated before the running maximum is
// moved and the accumulators rescaled: every P is then <= 2^15, inside the
// fp16 range, and the sums stay far from fp32 overflow.
constexpr float kSumLimit = 32768.0f;
// Running maximum before any key has been seen.  Finite, so that a masked
// score (-inf) minus it stays -inf (P = 0) instead of becoming NaN, while any
// visible score minus it overflows and forces the first real maximum in.
constexpr float kNoMax = -3.402823466e38f;
// Immediate of s_waitcnt vmcnt(n) with the other counters left alone.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// ---------------------------------------------------------------------------
// Element-type traits for the 16-bit MFMA path.
template <typename T> struct Ops;

template <> struct Ops<__bf16> {
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Two fp32 -> two bf16 (round to nearest even), packed in one dword.
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 r = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  // Row sums of P are taken from the fp32 values (bf16 rounding is too
  // coarse for the logsumexp).
  static constexpr bool kSumRounded = false;
};

template <> struct Ops<_Float16> {
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    f16x2 r = __builtin_convertvector(f, f16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  // Row sums of P may be taken from the packed fp16 values: acc + lo + hi
  // in one v_dot2_f32_f16 (products with 1.0 are exact, the sum is fp32).
  static constexpr bool kSumRounded = true;
  static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
  }
};

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: the
// two results hold, in every lane, the values of lanes l and l ^ 32).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over `bytes` bytes from `base`: loads at offsets >= bytes
// return zeros, so ragged tails need no clamping.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane buffer load straight into LDS: lane L's bytes land at
// lds_dst + 16 * L (lds_dst is wave-uniform).  The host pass of hipcc drops
// any kernel that names this builtin, so its body is compiled for the device
// pass only (the host pass never runs device code).
__device__ __forceinline__ void lds_load16(rsrc_t r, char* lds_dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, 0, 0, 0);
#else
  (void)r; (void)lds_dst; (void)voff;
#endif
}

// LDS tile layouts, cut into 16-byte chunks.  gfx950 LDS serves 256 bytes per
// cycle (64 four-byte banks); a ds_read_b128 takes 16 lanes per cycle.  Chunk
// c of row r is stored at chunk position c ^ swizzle(r), chosen so that the 16
// lanes of one cycle (one chunk of 16 consecutive rows) hit 16 different
// 16-byte bank groups.
//  K tile: 64 key rows x D values (2*D bytes per row):
//    D = 128: c ^ (r % 16);          D = 64: c ^ ((r / 2) % 8)
//  V^T tile: D rows (one per output column) x 64 keys (128 bytes per row):
//    c ^ ((r / 2) % 8)
template <bool B> struct BoolTag { static constexpr bool value = B; };

// Row-major 16-bit tiles that are read both by rows (one 16-byte
// ds_read_b128 per lane; 16 lanes, 16 consecutive rows, per cycle) and
// transposed (ds_read_b64_tr_b16; 32 lanes per cycle, 64 bytes from each of
// 4 consecutive rows): chunk c of row r is stored at chunk c ^ rm_swz(r),
// which keeps both patterns free of bank conflicts:
//   D = 128 (16 chunks per row): 4 * (r % 4) + (r / 4) % 4
//   D = 64  (8 chunks per row):  with m = (r / 2) % 8, 4 * (m % 2) + m / 2
// It has period 16 in r, and rm_swz(r + 8) = rm_swz(r) ^ 2 for r % 16 < 8.
template <int D>
__device__ __forceinline__ int rm_swz(int r) {
  if (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  const int m = (r >> 1) & 7;
  return 4 * (m & 1) + (m >> 1);
}

// Transposed MFMA A operand from a row-major rm_swz tile: for a 16-row
// chunk starting at row R (R % 16 == 0) and output columns 32 cb .. 32 cb
// + 31, lane L gets column 32 cb + L % 32 at the chunk's rows in the order
// of a 32x32x16 A operand's k index (k = 8 (L / 32) + j holds row
// 8 (j / 4) + 4 (L / 32) + j % 4, the order in which a 32x32 accumulator
// holds its rows).  ds_read_b64_tr_b16 gives output lane j of each 16-lane
// group element k of source lane 4 k + j / 4, element j % 4 (probed on
// gfx950), so source lane L reads 4 columns of row 4 (L / 32) + (L % 16) / 4
// (+ 8 for the second read).  tr_base is the per-lane byte offset of the
// first read for column block cb; the second read is at (tr_base ^ 32) + 8
// rows (rm_swz(r + 8) = rm_swz(r) ^ 2 flips bit 1 of the chunk index).
// The two transposing reads of one A operand (lo: first 8 rows, hi: the
// next 8), concatenated.  Device pass only, as lds_load16.
template <typename VEC8>
__device__ __forceinline__ VEC8 lds_read_tr(const char* lo, const char* hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  return __builtin_bit_cast(VEC8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
#else
  (void)lo; (void)hi;
  return VEC8{};
#endif
}

template <int D>
__device__ __forceinline__ int tr_base(int lane, int cb) {
  constexpr int RB = 2 * D;
  const int row_l = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int chunk_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return row_l * RB + (((4 * cb + chunk_l) ^ rm_swz<D>(row_l)) << 4) + 8 * (lane & 1);
}

template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int vt_swz(int r) { return (r >> 1) & 7; }

// Key stored at position j (0..15) of a 16-key group of a V^T row: the
// order of P^T's B-operand fragment (lanes 0-31 hold keys 0-3 and 8-11,
// lanes 32-63 keys 4-7 and 12-15), so one 16-byte read per lane is the A
// operand of O^T = V^T P^T.
__device__ __forceinline__ int vt_key(int j) {
  return (j & 3) | ((j & 4) << 1) | ((j & 8) >> 1);
}

}  // namespace fa

#endif  // FA_DEVICE_H
