// Host-only driver of the argument checks (fa_validate.cpp) for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer: a table of cases with
// known outcomes, then a deterministic sweep of extreme and random
// arguments (sizes near the 32- and 64-bit limits, odd addresses, NaN and
// infinite scales) through every check, so that an overflow or an
// out-of-bounds read in the checks is reported by the sanitizers.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "fa.h"
#include "fa_internal.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

const void* P(uintptr_t a) { return reinterpret_cast<const void*>(a); }

// xorshift64*: a fixed pseudo-random sequence.
uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}

int pick_int() {
  static const int edges[] = {0, 1, -1, 2, 63, 64, 65, 128, 4096, 32768, 1 << 20,
                              std::numeric_limits<int>::max(),
                              std::numeric_limits<int>::min(), 1 << 30, 7, 96};
  const uint64_t r = next();
  if (r % 3 == 0) return edges[(r >> 8) % (sizeof(edges) / sizeof(edges[0]))];
  return (int)(int64_t)(next() % 70000) - 100;
}

uintptr_t pick_addr() {
  static const uintptr_t edges[] = {0, 16, 0x100000, 0x100008, 0x100004, UINTPTR_MAX - 15,
                                    (uintptr_t)1 << 47, 0x200000};
  const uint64_t r = next();
  if (r % 2 == 0) return edges[(r >> 8) % (sizeof(edges) / sizeof(edges[0]))];
  return (uintptr_t)(next() & 0x0000FFFFFFFFFFF0ull);
}

float pick_scale() {
  static const float edges[] = {0.125f, 0.0f, -0.0f, -1.0f, 1e30f,
                                std::numeric_limits<float>::quiet_NaN(),
                                std::numeric_limits<float>::infinity(),
                                -std::numeric_limits<float>::infinity(),
                                std::numeric_limits<float>::denorm_min()};
  return edges[next() % (sizeof(edges) / sizeof(edges[0]))];
}

}  // namespace

int main() {
  using namespace fa;
  // Known outcomes (the layout of a small GQA launch at fake, aligned,
  // non-overlapping addresses; the checks never dereference them).
  const uintptr_t q = 0x100000, k = 0x200000, v = 0x300000, o = 0x400000, l = 0x500000;
  auto base = [&](float scale, int d, int dt, uintptr_t oo) {
    return check_args(P(q), P(k), P(v), P(oo), (const float*)P(l), 2, 8, 2, 64, 64, d, 1, scale,
                      nullptr, nullptr, dt, FA_F32);
  };
  expect("valid", base(0.125f, 128, FA_BF16, o), FA_OK);
  expect("negative scale", base(-0.5f, 128, FA_BF16, o), FA_OK);
  expect("zero scale", base(0.0f, 128, FA_BF16, o), FA_OK);
  expect("nan scale", base(std::nanf(""), 128, FA_BF16, o), FA_ERR_SCALE);
  expect("head dim", base(0.125f, 96, FA_BF16, o), FA_ERR_HEADDIM);
  expect("dtype", base(0.125f, 128, 9, o), FA_ERR_DTYPE);
  expect("alias", base(0.125f, 128, FA_BF16, v + 4096), FA_ERR_ALIAS);
  expect("align", base(0.125f, 128, FA_BF16, o + 8), FA_ERR_ALIGN);
  const int cu_ok[] = {0, 5, 5, 12};
  const int cu_bad[] = {0, 5, 4, 12};
  expect("seqlens ok", check_seqlens(cu_ok, 3, 7), FA_OK);
  expect("seqlens bad", check_seqlens(cu_bad, 3, 7), FA_ERR_SEQLENS);
  expect("seqlens long", check_seqlens(cu_ok, 3, 6), FA_ERR_SEQLENS);
  const int cu_wrap[] = {0, std::numeric_limits<int>::max(), std::numeric_limits<int>::min()};
  expect("seqlens wrap", check_seqlens(cu_wrap, 2, std::numeric_limits<int>::max()),
         FA_ERR_SEQLENS);

  // Sweep: every check with extreme and random arguments.  Only the
  // absence of sanitizer reports (and of crashes) is asserted here.
  uint64_t sum = 0;
  for (int it = 0; it < 200000; ++it) {
    const int B = pick_int(), Hq = pick_int(), Hkv = pick_int(), Nq = pick_int(),
              Nk = pick_int();
    const int d = (next() & 1) ? 128 : pick_int();
    const int causal = (int)(next() % 3), dt = (int)(next() % 4), odt = (int)(next() % 4);
    const float scale = pick_scale();
    const int* cuq = (next() & 1) ? (const int*)P(pick_addr()) : nullptr;
    const int* cuk = (next() & 3) ? cuq : (const int*)P(pick_addr());
    sum += (uint64_t)(check_args(P(pick_addr()), P(pick_addr()), P(pick_addr()),
                                 P(pick_addr()), (const float*)P(pick_addr()), B, Hq, Hkv, Nq,
                                 Nk, d, causal, scale, cuq, cuk, dt, odt) + 100);
    sum += (uint64_t)(check_packed_args(P(pick_addr()), P(pick_addr()), P(pick_addr()),
                                        next(), P(pick_addr()), (const float*)P(pick_addr()),
                                        B, Hq, Hkv, Nq, Nk, d, causal, scale, cuq, cuk, dt,
                                        odt) + 100);
    sum += (uint64_t)(check_pack_args(P(pick_addr()), P(pick_addr()), next(), B, Hkv, Nk, d,
                                      cuq, dt) + 100);
    sum += (uint64_t)(check_split_args(P(pick_addr()), next(), P(pick_addr()),
                                       (const float*)P(pick_addr()), B, Hq, Hkv, Nq, Nk, d,
                                       pick_int(), dt, odt, cuq != nullptr) + 100);
    sum += (uint64_t)(check_sparse_args(P(pick_addr()), pick_int(), pick_int(), P(pick_addr()),
                                        (const float*)P(pick_addr()), B, Hq, Nq, Nk, d, dt,
                                        odt, cuq != nullptr) + 100);
    BwdArgs a{P(pick_addr()), P(pick_addr()), P(pick_addr()), P(pick_addr()),
              P(pick_addr()), (const float*)P(pick_addr()), (void*)pick_addr(),
              (void*)pick_addr(), (void*)pick_addr(), cuq, B, Hq, Hkv, Nq, d, causal, scale,
              dt, odt, (int)(next() % 4), (void*)pick_addr()};
    sum += (uint64_t)(check_bwd_args(a, next()) + 100);
    sum += workspace_bytes(B, Hkv, Nk, d, dt) & 0xff;
    sum += split_workspace_bytes(B, Hq, Nq, d, pick_int()) & 0xff;
    sum += sparse_mask_bytes(pick_int(), pick_int(), Nq, Nk) & 0xff;
    sum += bwd_workspace_bytes(B, Hq, Hkv, Nq, d) & 0xff;
    sum += grid_size(B > 0 ? B : 1, Hq > 0 ? Hq : 1, Hkv > 0 ? Hkv : 1, Nq > 0 ? Nq : 1, d,
                     dt) & 0xff;
  }
  std::printf("sweep checksum %llu\n", (unsigned long long)sum);
  if (failures) return 1;
  std::printf("VALIDATE_SANITIZED_OK\n");
  return 0;
}
