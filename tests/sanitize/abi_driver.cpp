// Error paths of every entry point in include/fa.h, for a host build of the C ABI under
// AddressSanitizer and UndefinedBehaviorSanitizer (built and run by test_abi_sanitized.py).
// Each call below must return its status on the host before any HIP call; the sanitizers
// report any out-of-bounds access, overflow or other undefined behaviour on the way. The
// exit status is the number of calls that returned an unexpected status.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    ++failures;
    fprintf(stderr, "FAIL %s: got %d (%s), want %d\n", what, got, fa_strerror(got), want);
  }
}

// a 16-byte aligned non-null address; failing calls never dereference it
void* const F = reinterpret_cast<void*>(uintptr_t{0x10000});
float* const FF = reinterpret_cast<float*>(uintptr_t{0x10000});
const int* const FI = reinterpret_cast<const int*>(uintptr_t{0x10000});
void* const MIS = reinterpret_cast<void*>(uintptr_t{0x10002});  // misaligned

constexpr int BF = FA_DTYPE_BF16, F32 = FA_DTYPE_F32;

}  // namespace

int main() {
  for (int code = -9; code <= 1; ++code)
    if (!fa_strerror(code) || strlen(fa_strerror(code)) == 0) expect(1, 0, "fa_strerror non-empty");

  // size queries: exact values, zero for negative sizes, no overflow at large sizes
  expect(fa_bwd_workspace_bytes(4, 16, 4096) == size_t(2) * 4 * 16 * 4096 * 4, 1, "bwd workspace bytes");
  expect(fa_bwd_workspace_bytes(-1, 1, 1) == 0, 1, "bwd workspace negative");
  expect(fa_decode_workspace_bytes(64, 32, 128, 64) == size_t(64) * 32 * 64 * 130 * 4, 1, "decode workspace");
  expect(fa_decode_workspace_bytes(1, -1, 128, 1) == 0, 1, "decode workspace negative");
  (void)fa_fwd_fp8_workspace_bytes(2, 16, 16, 8192, 128);
  (void)fa_fwd_fp8_workspace_bytes(1 << 30, 1 << 10, 1 << 10, 1 << 30, 128);
  (void)fa_decode_workspace_bytes(1 << 30, 1 << 30, 1 << 30, 1 << 30);

  // fa_fwd
  expect(fa_fwd(F, F, F, F, FF, -1, 1, 1, 16, 64, 0.125f, 0, BF, nullptr), FA_ERR_SHAPE, "fwd B<0");
  expect(fa_fwd(F, F, F, F, FF, 1, 6, 4, 16, 64, 0.125f, 0, BF, nullptr), FA_ERR_SHAPE, "fwd H%Hkv");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 96, 0.125f, 0, BF, nullptr), FA_ERR_HEADDIM, "fwd d=96");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 64, 0.125f, 0, 7, nullptr), FA_ERR_DTYPE, "fwd dtype");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 64, NAN, 0, BF, nullptr), FA_ERR_ARG, "fwd scale NaN");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 64, INFINITY, 0, BF, nullptr), FA_ERR_ARG, "fwd scale inf");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 64, -1.f, 0, BF, nullptr), FA_ERR_ARG, "fwd scale<0");
  expect(fa_fwd(F, F, F, F, FF, 1, 1, 1, 16, 64, 0.125f, 2, BF, nullptr), FA_ERR_ARG, "fwd causal=2");
  expect(fa_fwd(nullptr, F, F, F, FF, 1, 1, 1, 16, 64, 0.125f, 0, BF, nullptr), FA_ERR_NULL, "fwd q NULL");
  expect(fa_fwd(F, F, F, MIS, FF, 1, 1, 1, 16, 64, 0.125f, 0, BF, nullptr), FA_ERR_ARG, "fwd o misaligned");
  expect(fa_fwd(F, F, F, F, FF, 1 << 30, 1 << 10, 1 << 10, 1 << 30, 64, 0.125f, 0, BF, nullptr), FA_ERR_SHAPE,
         "fwd too large");
  expect(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 16, 64, 0.125f, 0, BF, nullptr), FA_OK,
         "fwd empty batch");

  // fa_fwd_window
  expect(fa_fwd_window(F, F, F, F, FF, 1, 2, 2, 16, 32, 128, 0.1f, 1, -2, -1, BF, nullptr), FA_ERR_ARG,
         "window left<-1");
  expect(fa_fwd_window(F, F, F, F, FF, 1, 2, 2, -16, 32, 128, 0.1f, 1, -1, -1, BF, nullptr), FA_ERR_SHAPE,
         "window Nq<0");
  // window offsets near the int range: the offset arithmetic runs (in 64 bits) before the
  // pointer check
  expect(fa_fwd_window(nullptr, F, F, F, FF, 1, 2, 2, 1 << 30, 1 << 30, 128, 0.1f, 0, 0x7fffffff, 0x7fffffff, BF,
                       nullptr), FA_ERR_NULL, "window huge offsets");

  // fa_fwd_varlen
  expect(fa_fwd_varlen(F, F, F, F, FF, FI, 2, 100, 200, 2, 2, 64, 0.1f, 1, BF, nullptr), FA_ERR_SHAPE,
         "varlen max_seqlen > total");
  expect(fa_fwd_varlen(F, F, F, F, FF, nullptr, 2, 100, 60, 2, 2, 64, 0.1f, 1, BF, nullptr), FA_ERR_NULL,
         "varlen cu NULL");
  expect(fa_fwd_varlen(F, F, F, F, FF, FI, 0, 100, 60, 2, 2, 64, 0.1f, 1, BF, nullptr), FA_ERR_SHAPE,
         "varlen no sequences");
  expect(fa_fwd_varlen(F, F, F, F, FF, FI, 2, (1 << 30) + 1, 60, 2, 2, 64, 0.1f, 1, BF, nullptr), FA_ERR_SHAPE,
         "varlen too many tokens");

  // fa_fwd_fp8
  expect(fa_fwd_fp8(F, F, F, nullptr, F, FF, 1, 4, 2, 100, 128, 0.1f, 1, F, 16, nullptr), FA_ERR_WORKSPACE,
         "fp8 workspace small");
  expect(fa_fwd_fp8(F, F, F, reinterpret_cast<const float*>(MIS), F, FF, 1, 4, 2, 100, 128, 0.1f, 1, F,
                    size_t(1) << 24, nullptr), FA_ERR_ARG,
         "fp8 signs misaligned");
  expect(fa_fwd_fp8(F, F, F, nullptr, F, FF, 1, 4, 2, 100, 96, 0.1f, 1, F, size_t(1) << 24, nullptr),
         FA_ERR_HEADDIM, "fp8 d=96");

  // fa_bwd
  expect(fa_bwd(F, F, F, F, FF, F, FF, FF, FF, 1, 2, 2, 100, 128, 0.1f, 1, F32, F, 1 << 20, nullptr), FA_ERR_DTYPE,
         "bwd fp32");
  expect(fa_bwd(F, F, F, F, FF, F, FF, FF, FF, 1, 2, 2, 100, 128, 0.1f, 1, BF, F, 16, nullptr), FA_ERR_WORKSPACE,
         "bwd workspace small");
  expect(fa_bwd(F, F, F, F, FF, F, nullptr, FF, FF, 1, 2, 2, 100, 128, 0.1f, 1, BF, F, 1 << 20, nullptr),
         FA_ERR_NULL, "bwd dq NULL");

  // fa_decode
  expect(fa_decode(F, F, F, F, nullptr, 2, 4, 4, 1000, 128, 0.1f, 0, BF, F, 1 << 20, nullptr), FA_ERR_ARG,
         "decode splits=0");
  expect(fa_decode(F, F, F, F, nullptr, 2, 4, 4, 1000, 128, 0.1f, 1025, BF, F, 1 << 20, nullptr), FA_ERR_ARG,
         "decode splits>1024");
  expect(fa_decode(F, F, F, F, nullptr, 2, 4, 4, 0, 128, 0.1f, 8, BF, F, 1 << 20, nullptr), FA_ERR_SHAPE,
         "decode L=0");
  expect(fa_decode(F, F, F, F, nullptr, 2, 4, 4, 1000, 128, 0.1f, 8, BF, F, 8191, nullptr), FA_ERR_WORKSPACE,
         "decode workspace small");

  // fa_decode_noalloc: the scratch limit is checked on the host, without overflow
  expect(fa_decode_noalloc(F, F, F, F, nullptr, 64, 32, 32, 32768, 128, 0.1f, 64, BF, nullptr), FA_ERR_SCRATCH,
         "noalloc over 64 MiB");
  expect(fa_decode_noalloc(F, F, F, F, nullptr, 1 << 20, 1 << 10, 1 << 10, 1, 128, 0.1f, 1024, BF, nullptr),
         FA_ERR_SCRATCH, "noalloc huge");
  expect(fa_decode_noalloc(nullptr, F, F, F, nullptr, 64, 32, 32, 32768, 128, 0.1f, 63, BF, nullptr), FA_ERR_NULL,
         "noalloc q NULL");
  expect(fa_decode_noalloc(F, F, F, F, nullptr, 2, 4, 3, 1000, 128, 0.1f, 8, BF, nullptr), FA_ERR_SHAPE,
         "noalloc H%Hkv");

  // fa_decode_paged
  expect(fa_decode_paged(F, F, F, FI, FI, F, nullptr, 2, 4, 2, 128, 24, 100, 20, 0.1f, 8, BF, F, 1 << 20, nullptr),
         FA_ERR_SHAPE, "paged page_size 24");
  expect(fa_decode_paged(F, F, F, FI, FI, F, nullptr, 2, 4, 2, 128, 16, 100, (1 << 26) + 1, 0.1f, 8, BF, F, 1 << 20,
                         nullptr), FA_ERR_SHAPE, "paged too many pages");
  expect(fa_decode_paged(F, F, F, reinterpret_cast<const int*>(uintptr_t{0x10002}), FI, F, nullptr, 2, 4, 2, 128,
                         16, 100, 20, 0.1f, 8, BF, F, 1 << 20, nullptr), FA_ERR_ARG, "paged table misaligned");

  if (failures) fprintf(stderr, "%d unexpected statuses\n", failures);
  else printf("all error paths returned their expected status\n");
  return failures;
}
