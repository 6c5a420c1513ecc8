// C ABI of libfa (declared and documented in include/fa.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"
#include "fa_poison.h"

namespace {

constexpr int kMaxDevices = 64;

// Per-device "is gfx950" answer, filled once per device.
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

// Compute units of the current device, 0 if unknown.
int device_cus() {
  int dev = -1, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return FA_ERR_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                    std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  return g_dev_ok[dev] ? FA_OK : FA_ERR_DEVICE;
}

// FA_DEBUG=1 in the environment (read once): packed offset arrays are
// checked on the device before any attention kernel runs.
bool debug_mode() {
  static const bool on = [] {
    const char* e = std::getenv("FA_DEBUG");
    return e != nullptr && std::strcmp(e, "1") == 0;
  }();
  return on;
}

// The debug check of the query and key offsets of a packed launch (no-op
// outside debug mode or for fixed-length layouts).
int debug_seqlens(const int* cu_q, const int* cu_k, int B, int Nq, int Nk, void* stream) {
  if (!debug_mode() || cu_q == nullptr) return FA_OK;
  int st = fa::debug_check_seqlens(cu_q, B, Nq, stream);
  if (st == FA_OK && cu_k != cu_q) st = fa::debug_check_seqlens(cu_k, B, Nk, stream);
  return st;
}

// The forced launch order: FA_FORCE_ORDER (-1 .. 3) at first use, then
// whatever fa_debug_force_order sets.
std::atomic<int>& order_setting() {
  static std::atomic<int> v{[] {
    const char* e = std::getenv("FA_FORCE_ORDER");
    if (e == nullptr) return -1;
    char* end = nullptr;
    const long x = std::strtol(e, &end, 10);
    return (end != e && *end == '\0' && x >= -1 && x <= 3) ? (int)x : -1;
  }()};
  return v;
}

}  // namespace

int fa::forced_order() { return order_setting().load(std::memory_order_relaxed); }

extern "C" {

int fa_debug_force_order(int order) {
  if (order < -1 || order > 3) return FA_ERR_SHAPE;
  order_setting().store(order, std::memory_order_relaxed);
  return FA_OK;
}

int fa_debug_forced_order(void) { return fa::forced_order(); }

int fa_build_flags(void) { return fa::kPoisonLds ? FA_BUILD_POISON_LDS : 0; }

int fa_fwd_check(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, int B, int Hq, int Hkv, int N, int d,
                 int causal, float scale, const int* cu_seqlens, int in_dtype,
                 int out_dtype) {
  return fa::check_args(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, scale,
                        cu_seqlens, cu_seqlens, in_dtype, out_dtype);
}

size_t fa_workspace_bytes(int B, int Hkv, int N, int d, int in_dtype) {
  if ((d != 64 && d != 128) || (in_dtype != FA_F16 && in_dtype != FA_BF16)) return 0;
  const uint64_t n = fa::workspace_bytes(B, Hkv, N, d, in_dtype);
  return n > (uint64_t)SIZE_MAX ? SIZE_MAX : (size_t)n;
}

int fa_pack_v(const void* v, void* vt, size_t vt_bytes, int B, int Hkv, int N, int d,
              const int* cu_seqlens, void* stream, int in_dtype) {
  int st = fa::check_pack_args(v, vt, vt_bytes, B, Hkv, N, d, cu_seqlens, in_dtype);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  return fa::launch_vt_pack(v, vt, B, Hkv, N, d, cu_seqlens, in_dtype, stream);
}

int fa_fwd_kv_packed(const void* q, const void* k, const void* vt, size_t vt_bytes, void* o,
                     float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                     float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
                     void* stream, int in_dtype, int out_dtype) {
  int st = fa::check_packed_args(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                                 scale, cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, nullptr, o, lse, vt, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  return fa::launch_fwd(a, stream);
}

int fa_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int in_dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv != 0 ||
      (d != 64 && d != 128))
    return 1;
  return fa::suggest_splits(B, Hq, Hkv, Nq, Nk, d, in_dtype, device_cus());
}

size_t fa_split_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits) {
  if (num_splits < 2) return 0;
  const uint64_t n = fa::split_workspace_bytes(B, Hq, Nq, d, num_splits);
  return n > (uint64_t)SIZE_MAX ? SIZE_MAX : (size_t)n;
}

int fa_fwd_kv_split_packed(const void* q, const void* k, const void* vt, size_t vt_bytes,
                           void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                           int causal, float scale, const int* cu_seqlens_q,
                           const int* cu_seqlens_k, int num_splits, void* part,
                           size_t part_bytes, void* stream, int in_dtype, int out_dtype) {
  int st = fa::check_packed_args(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                                 scale, cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = fa::check_split_args(part, part_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, num_splits,
                            in_dtype, out_dtype, cu_seqlens_q != nullptr);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, nullptr, o, lse, vt, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  if (num_splits > 1) {
    a.n_splits = num_splits;
    a.o_part = (float*)part;
    a.lse_part = (float*)((char*)part + (size_t)num_splits * B * Hq * Nq * d * 4);
  }
  return fa::launch_fwd(a, stream);
}

int fa_fwd_kv_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            float scale, const int* cu_seqlens_q, const int* cu_seqlens_k,
                            int num_splits, void* stream, int in_dtype, int out_dtype) {
  int st = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                          cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  if (in_dtype == FA_F32) return FA_ERR_DTYPE;
  if (num_splits < 1 || num_splits > 256) return FA_ERR_SHAPE;
  const uint64_t need = num_splits > 1 ? fa::split_workspace_bytes(B, Hq, Nq, d, num_splits) : 0;
  if (need > fa::kNoAllocScratchBytes) return FA_ERR_SCRATCH;
  st = device_status();
  if (st != FA_OK) return st;
  void* part = nullptr;
  if (num_splits > 1) {
    part = fa::noalloc_scratch();
    if (!part) return FA_ERR_DEVICE;
  }
  st = fa::check_split_args(part, need, o, lse, B, Hq, Hkv, Nq, Nk, d, num_splits, in_dtype,
                            out_dtype, cu_seqlens_q != nullptr);
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, v, o, lse, nullptr, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  if (num_splits > 1) {
    a.n_splits = num_splits;
    a.o_part = (float*)part;
    a.lse_part = (float*)((char*)part + (size_t)num_splits * B * Hq * Nq * d * 4);
  }
  return fa::launch_fwd(a, stream);
}

size_t fa_noalloc_scratch_bytes(void) { return (size_t)fa::kNoAllocScratchBytes; }

int fa_fwd_packed(const void* q, const void* k, const void* vt, size_t vt_bytes, void* o,
                  float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                  const int* cu_seqlens, void* stream, int in_dtype, int out_dtype) {
  return fa_fwd_kv_packed(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, N, N, d, causal, scale,
                          cu_seqlens, cu_seqlens, stream, in_dtype, out_dtype);
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream,
              int in_dtype, int out_dtype) {
  // One kernel launch reading q, k, v and writing o, lse; no workspace.
  int st = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                          cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, v, o, lse, nullptr, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  return fa::launch_fwd(a, stream);
}

int fa_fwd_kv_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_splits,
                    void* part, size_t part_bytes, void* stream, int in_dtype, int out_dtype) {
  int st = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                          cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  if (in_dtype == FA_F32) return FA_ERR_DTYPE;
  st = fa::check_split_args(part, part_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, num_splits,
                            in_dtype, out_dtype, cu_seqlens_q != nullptr);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, v, o, lse, nullptr, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  if (num_splits > 1) {
    a.n_splits = num_splits;
    a.o_part = (float*)part;
    a.lse_part = (float*)((char*)part + (size_t)num_splits * B * Hq * Nq * d * 4);
  }
  return fa::launch_fwd(a, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           const int* cu_seqlens, void* stream, int in_dtype, int out_dtype) {
  return fa_fwd_kv(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, scale, cu_seqlens,
                   cu_seqlens, stream, in_dtype, out_dtype);
}

int fa_fwd_sparse_packed(const void* q, const void* k, const void* vt, size_t vt_bytes,
                         void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         int causal, float scale, const int* cu_seqlens_q,
                         const int* cu_seqlens_k, const unsigned char* block_mask,
                         int mask_batches, int mask_heads, void* stream, int in_dtype,
                         int out_dtype) {
  int st = fa::check_packed_args(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                                 scale, cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = fa::check_sparse_args(block_mask, mask_batches, mask_heads, o, lse, B, Hq, Nq, Nk, d,
                             in_dtype, out_dtype, cu_seqlens_q != nullptr);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, nullptr, o, lse, vt, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  a.block_mask = block_mask;
  a.mask_batches = mask_batches;
  a.mask_heads = mask_heads;
  return fa::launch_fwd(a, stream);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  const unsigned char* block_mask, int mask_batches, int mask_heads,
                  void* stream, int in_dtype, int out_dtype) {
  int st = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                          cu_seqlens_q, cu_seqlens_k, in_dtype, out_dtype);
  if (st != FA_OK) return st;
  st = fa::check_sparse_args(block_mask, mask_batches, mask_heads, o, lse, B, Hq, Nq, Nk, d,
                             in_dtype, out_dtype, cu_seqlens_q != nullptr);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens_q, cu_seqlens_k, B, Nq, Nk, stream);
  if (st != FA_OK) return st;
  fa::LaunchArgs a{q, k, v, o, lse, nullptr, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Nq, Nk,
                   d, causal, scale, in_dtype, out_dtype};
  a.block_mask = block_mask;
  a.mask_batches = mask_batches;
  a.mask_heads = mask_heads;
  return fa::launch_fwd(a, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int in_dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || (d != 64 && d != 128) ||
      (in_dtype != FA_F16 && in_dtype != FA_BF16))
    return 0;
  const uint64_t n = fa::bwd_workspace_bytes(B, Hq, Hkv, N, d);
  return n > (uint64_t)SIZE_MAX ? SIZE_MAX : (size_t)n;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
           int causal, float scale, const int* cu_seqlens, void* workspace,
           size_t workspace_bytes, void* stream, int in_dtype, int o_dtype, int grad_dtype) {
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, Hq, Hkv, N, d, causal,
                scale, in_dtype, o_dtype, grad_dtype, workspace};
  int st = fa::check_bwd_args(a, workspace_bytes);
  if (st != FA_OK) return st;
  st = device_status();
  if (st != FA_OK) return st;
  st = debug_seqlens(cu_seqlens, cu_seqlens, B, N, N, stream);
  if (st != FA_OK) return st;
  return fa::launch_bwd(a, stream);
}

const char* fa_kernel_name(int in_dtype, int d, int causal, int varlen,
                           int out_dtype) {
  return fa::kernel_name(in_dtype, d, causal, varlen, out_dtype);
}

const char* fa_kernel_name_kv(int in_dtype, int d, int causal, int varlen, int out_dtype,
                              int Hq, int Hkv, int Nq) {
  if (Hkv < 1 || Hq < 1 || Nq < 1) return nullptr;
  return fa::kernel_name_kv(in_dtype, d, causal, varlen, out_dtype, Hq, Hkv, Nq);
}

const char* fa_kernel_name_ex(int in_dtype, int d, int causal, int varlen, int out_dtype,
                              int Hq, int Hkv, int Nq, int sparse, int vt_packed) {
  if (Hkv < 1 || Hq < 1 || Nq < 1) return nullptr;
  return fa::kernel_name_kv(in_dtype, d, causal, varlen, out_dtype, Hq, Hkv, Nq, sparse,
                            vt_packed);
}

int fa_check_seqlens(const int* cu_seqlens, int B, int n_max) {
  if (B < 0) return FA_ERR_SHAPE;
  return fa::check_seqlens(cu_seqlens, B, n_max);
}

int fa_supported(int in_dtype, int d, int causal) {
  const bool dt = in_dtype == FA_F32 || in_dtype == FA_F16 || in_dtype == FA_BF16;
  return dt && (d == 64 || d == 128) && (causal == 0 || causal == 1);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "bad shape: B, Hq, Hkv, N must be >= 1, causal 0 or 1, sizes in range";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_GQA: return "Hq must be a multiple of Hkv";
    case FA_ERR_DTYPE: return "bad dtype: in_dtype F32/F16/BF16, out_dtype F32 or in_dtype";
    case FA_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes, lse and cu_seqlens 4";
    case FA_ERR_ALIAS: return "o overlaps q, k, v or lse";
    case FA_ERR_SCALE: return "scale must be finite (and > 0 for the backward)";
    case FA_ERR_DEVICE: return "no usable device: the current HIP device is not gfx950";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace too small: see fa_workspace_bytes";
    case FA_ERR_ALLOC: return "could not allocate device memory (no entry point allocates)";
    case FA_ERR_SEQLENS: return "corrupt cu_seqlens: cu[0] != 0, decreasing, or a length above N";
    case FA_ERR_SCRATCH: return "split-KV partials exceed the library's fixed scratch "
                                "(fa_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

int fa_version(void) { return 1 * 10000 + 2 * 100 + 0; }

}  // extern "C"
