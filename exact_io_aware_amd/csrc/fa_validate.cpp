// Argument checks of the attention entry points and fa_pack_v (include/fa.h).  Pure C++: no HIP call, so the
// checks run, and are tested, on a machine without a GPU.
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_internal.h"

namespace fa {

namespace {

size_t elem_size(int dt) { return dt == FA_F32 ? 4 : 2; }

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool overlap(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb) {
  return a < b + nb && b < a + na;
}

}  // namespace

int check_args(const void* q, const void* k, const void* v, const void* o,
               const float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
               int in_dtype, int out_dtype, uint64_t v_bytes) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if ((cu_seqlens_q == nullptr) != (cu_seqlens_k == nullptr)) return FA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || (causal != 0 && causal != 1))
    return FA_ERR_SHAPE;
  if (Nq > kMaxSeqLen || Nk > kMaxSeqLen) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if (in_dtype != FA_F32 && in_dtype != FA_F16 && in_dtype != FA_BF16)
    return FA_ERR_DTYPE;
  if (out_dtype != FA_F32 && out_dtype != in_dtype) return FA_ERR_DTYPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;

  // Element counts; the packed layout's token counts are bounded by B * Nq
  // and B * Nk.
  uint64_t rows, krows, qn, kn, ln;
  if (!mul_ok((uint64_t)B, (uint64_t)Nq, &rows)) return FA_ERR_SHAPE;
  if (!mul_ok((uint64_t)B, (uint64_t)Nk, &krows)) return FA_ERR_SHAPE;
  if (!mul_ok(rows, (uint64_t)Hq * (uint64_t)d, &qn)) return FA_ERR_SHAPE;
  if (!mul_ok(krows, (uint64_t)Hkv * (uint64_t)d, &kn)) return FA_ERR_SHAPE;
  if (!mul_ok(rows, (uint64_t)Hq, &ln)) return FA_ERR_SHAPE;
  if (v_bytes == 0) v_bytes = kn * elem_size(in_dtype);
  // Kernel index arithmetic uses 64-bit element offsets and 32-bit row,
  // head and workgroup counts.
  if (qn > (uint64_t)INT64_MAX / 4 || kn > (uint64_t)INT64_MAX / 4 ||
      ln > (uint64_t)INT32_MAX * 64)
    return FA_ERR_SHAPE;
  if (grid_size(B, Hq, Hkv, Nq, d, in_dtype) > (uint64_t)INT32_MAX)
    return FA_ERR_SHAPE;

  auto mis = [](const void* p, uintptr_t a) { return ((uintptr_t)p) % a != 0; };
  if (mis(q, 16) || mis(k, 16) || mis(v, 16) || mis(o, 16) || mis(lse, 4) ||
      (cu_seqlens_q && mis(cu_seqlens_q, 4)) || (cu_seqlens_k && mis(cu_seqlens_k, 4)))
    return FA_ERR_ALIGN;

  // o must not overlap any input or lse.  For the packed layout the true
  // extent (T tokens) lives on the device, so only the B*N bound is known:
  // there only identical start pointers are rejected.
  const uintptr_t po = (uintptr_t)o;
  if (po == (uintptr_t)q || po == (uintptr_t)k || po == (uintptr_t)v ||
      po == (uintptr_t)lse)
    return FA_ERR_ALIAS;
  if (!cu_seqlens_q) {
    const uint64_t ob = qn * elem_size(out_dtype), ib = elem_size(in_dtype);
    if (overlap(po, ob, (uintptr_t)q, qn * ib) ||
        overlap(po, ob, (uintptr_t)k, kn * ib) ||
        overlap(po, ob, (uintptr_t)v, v_bytes) ||
        overlap(po, ob, (uintptr_t)lse, ln * 4))
      return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int check_packed_args(const void* q, const void* k, const void* vt, uint64_t vt_bytes,
                      const void* o, const float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                      int d, int causal, float scale, const int* cu_seqlens_q,
                      const int* cu_seqlens_k, int in_dtype, int out_dtype) {
  if (in_dtype == FA_F32) return FA_ERR_DTYPE;   // fp32 inputs use V itself
  const uint64_t need = workspace_bytes(B, Hkv, Nk, d, in_dtype);
  const int st = check_args(q, k, vt, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                            cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype, need);
  if (st != FA_OK) return st;
  if (vt_bytes < need) return FA_ERR_WORKSPACE;
  if (need / (128ull * (uint64_t)d) > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_split_args(const void* part, uint64_t part_bytes, const void* o, const float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits,
                     int in_dtype, int out_dtype, bool varlen) {
  (void)Nk;
  if (num_splits < 1 || num_splits > 256) return FA_ERR_SHAPE;
  if (num_splits == 1) return FA_OK;
  if (!part) return FA_ERR_NULL;
  if (((uintptr_t)part) % 16 != 0) return FA_ERR_ALIGN;
  const uint64_t need = split_workspace_bytes(B, Hq, Nq, d, num_splits);
  if (part_bytes < need) return FA_ERR_WORKSPACE;
  if (grid_size(B, Hq, Hkv, Nq, d, in_dtype) * (uint64_t)num_splits > (uint64_t)INT32_MAX)
    return FA_ERR_SHAPE;
  uint64_t rows;
  if (!mul_ok((uint64_t)B * (uint64_t)Hq, (uint64_t)Nq, &rows)) return FA_ERR_SHAPE;
  // For the packed layout o's true extent (Tq rows) lives on the device:
  // only identical start pointers are rejected there.
  const uint64_t ob = varlen ? 1 : rows * (uint64_t)d * elem_size(out_dtype);
  if (overlap((uintptr_t)part, need, (uintptr_t)o, ob) ||
      overlap((uintptr_t)part, need, (uintptr_t)lse, rows * 4))
    return FA_ERR_ALIAS;
  return FA_OK;
}

uint64_t sparse_mask_bytes(int mask_batches, int mask_heads, int Nq, int Nk) {
  const uint64_t nqb = ((uint64_t)Nq + kSparseBlock - 1) / kSparseBlock;
  const uint64_t nkb = ((uint64_t)Nk + kSparseBlock - 1) / kSparseBlock;
  uint64_t n;
  if (!mul_ok((uint64_t)mask_batches * (uint64_t)mask_heads, nqb * nkb, &n)) return UINT64_MAX;
  return n;
}

int check_sparse_args(const void* block_mask, int mask_batches, int mask_heads, const void* o,
                      const float* lse, int B, int Hq, int Nq, int Nk, int d, int in_dtype,
                      int out_dtype, bool varlen) {
  if (!block_mask) return FA_ERR_NULL;
  if (in_dtype == FA_F32) return FA_ERR_DTYPE;
  if ((mask_batches != 1 && mask_batches != B) || (mask_heads != 1 && mask_heads != Hq))
    return FA_ERR_SHAPE;
  if (((uint64_t)Nk + kSparseBlock - 1) / kSparseBlock > (uint64_t)kMaxSparseTiles)
    return FA_ERR_SHAPE;
  const uint64_t mb = sparse_mask_bytes(mask_batches, mask_heads, Nq, Nk);
  if (mb > (uint64_t)INT64_MAX / 2) return FA_ERR_SHAPE;
  // The mask is an input: it must not overlap the outputs.  For the packed
  // layout o's true extent lives on the device (only the start is checked).
  uint64_t rows = (uint64_t)B * (uint64_t)Hq * (uint64_t)Nq;
  const uint64_t ob = varlen ? 1 : rows * (uint64_t)d * elem_size(out_dtype);
  if (block_mask == o || overlap((uintptr_t)block_mask, mb, (uintptr_t)o, ob) ||
      overlap((uintptr_t)block_mask, mb, (uintptr_t)lse, rows * 4))
    return FA_ERR_ALIAS;
  return FA_OK;
}

int check_bwd_args(const BwdArgs& a, uint64_t ws_bytes) {
  if (!a.q || !a.k || !a.v || !a.o || !a.dout || !a.lse || !a.dq || !a.dk || !a.dv ||
      !a.workspace)
    return FA_ERR_NULL;
  // The forward's checks cover shapes, head dim, GQA, scale, alignment of
  // q, k, v, o and lse, and o against the inputs.
  const int st = check_args(a.q, a.k, a.v, a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, a.N, a.d, a.causal,
                            a.scale, a.cu_seqlens, a.cu_seqlens, a.in_dtype, a.o_dtype);
  if (st != FA_OK) return st;
  // The backward kernels take the scale as given (no sign folding).
  if (!(a.scale > 0.0f)) return FA_ERR_SCALE;
  if (a.in_dtype == FA_F32) return FA_ERR_DTYPE;
  if (a.grad_dtype != FA_F32 && a.grad_dtype != a.in_dtype) return FA_ERR_DTYPE;
  auto mis = [](const void* p, uintptr_t al) { return ((uintptr_t)p) % al != 0; };
  if (mis(a.dout, 16) || mis(a.dq, 16) || mis(a.dk, 16) || mis(a.dv, 16) ||
      mis(a.workspace, 16))
    return FA_ERR_ALIGN;
  if (ws_bytes < bwd_workspace_bytes(a.B, a.Hq, a.Hkv, a.N, a.d)) return FA_ERR_WORKSPACE;
  if (grid_size(a.B, a.Hq, a.Hkv, a.N, a.d, a.in_dtype) > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  // Outputs must not overlap each other, the inputs or the workspace.  For
  // the packed layout only identical start pointers are rejected.
  const uint64_t qn = (uint64_t)a.B * a.N * a.Hq * a.d, kn = (uint64_t)a.B * a.N * a.Hkv * a.d;
  const uint64_t gs = elem_size(a.grad_dtype), is = elem_size(a.in_dtype);
  const bool fixed = a.cu_seqlens == nullptr;
  struct R { const void* p; uint64_t n; };
  const R outs[3] = {{a.dq, fixed ? qn * gs : 1}, {a.dk, fixed ? kn * gs : 1},
                     {a.dv, fixed ? kn * gs : 1}};
  const R ins[7] = {{a.q, fixed ? qn * is : 1}, {a.k, fixed ? kn * is : 1},
                    {a.v, fixed ? kn * is : 1}, {a.o, fixed ? qn * elem_size(a.o_dtype) : 1},
                    {a.dout, fixed ? qn * is : 1},
                    {a.lse, (uint64_t)a.B * a.Hq * a.N * 4}, {a.workspace, ws_bytes}};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (outs[i].p == ins[j].p ||
          overlap((uintptr_t)outs[i].p, outs[i].n, (uintptr_t)ins[j].p, ins[j].n))
        return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (outs[i].p == outs[j].p ||
          overlap((uintptr_t)outs[i].p, outs[i].n, (uintptr_t)outs[j].p, outs[j].n))
        return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int check_pack_args(const void* v, const void* vt, uint64_t vt_bytes, int B, int Hkv, int N,
                    int d, const int* cu_seqlens, int in_dtype) {
  if (!v || !vt) return FA_ERR_NULL;
  if (B < 1 || Hkv < 1 || N < 1 || N > kMaxSeqLen) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_DTYPE;
  uint64_t rows, vn;
  if (!mul_ok((uint64_t)B, (uint64_t)N, &rows)) return FA_ERR_SHAPE;
  if (!mul_ok(rows, (uint64_t)Hkv * (uint64_t)d, &vn)) return FA_ERR_SHAPE;
  if (vn > (uint64_t)INT64_MAX / 4) return FA_ERR_SHAPE;
  const uint64_t need = workspace_bytes(B, Hkv, N, d, in_dtype);
  // One workgroup per tile, counted in 32 bits.
  if (need / (128ull * (uint64_t)d) > (uint64_t)INT32_MAX) return FA_ERR_SHAPE;
  auto mis = [](const void* p, uintptr_t a) { return ((uintptr_t)p) % a != 0; };
  if (mis(v, 16) || mis(vt, 16) || (cu_seqlens && mis(cu_seqlens, 4))) return FA_ERR_ALIGN;
  if (vt_bytes < need) return FA_ERR_WORKSPACE;
  if ((uintptr_t)vt == (uintptr_t)v ||
      (!cu_seqlens && overlap((uintptr_t)vt, need, (uintptr_t)v, vn * 2)))
    return FA_ERR_ALIAS;
  return FA_OK;
}

}  // namespace fa
