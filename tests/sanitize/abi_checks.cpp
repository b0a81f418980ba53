// Host-side checks of libkla's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Every call below must be
// settled by the library's validation or planning before any kernel is enqueued:
// the kernel launchers are linked as stubs that abort (launch_stubs.cpp), so a
// call that slips past validation ends the run. Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kla.h"

static int failures = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static void* const P = reinterpret_cast<void*>(0x1000);   // never dereferenced
static float* const F = reinterpret_cast<float*>(0x2000);
static float* const MIS = reinterpret_cast<float*>(0x2008);  // 8-byte aligned only

static bool has_error_text() { return std::strlen(kla_last_error()) > 0; }

int main() {
  // prefill: sizes, nulls, modes, alignment
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 0, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(has_error_text());
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, -5, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 96, 64, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 256, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 64, 32, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd(nullptr, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, nullptr, nullptr, 1, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd(P, P, P, MIS, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(std::strstr(kla_last_error(), "16-byte") != nullptr);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 70000, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1 << 20, 128, 128, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd_f32(F, F, F, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 256, 64, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  // T == 0 without a final state: nothing to do, nothing enqueued
  CHECK(kla_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 1e-6f, nullptr, nullptr, nullptr, 2, 0, 3, 64, 64, 64,
                      nullptr) == KLA_OK);
  CHECK(kla_chunk_fwd_ex(static_cast<kla_dtype>(9), KLA_BETA_KACZMARZ, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1,
                         64, 64, 64, KLA_PATH_AUTO, 0, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd_ex(KLA_DTYPE_BF16, static_cast<kla_beta_mode>(5), P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64,
                         1, 64, 64, 64, KLA_PATH_AUTO, 0, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd_ex(KLA_DTYPE_BF16, KLA_BETA_DIRECT, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 64, 64,
                         static_cast<kla_path>(7), 0, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd_ex(KLA_DTYPE_BF16, KLA_BETA_DIRECT, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 64, 64, 64,
                         KLA_PATH_SCAN, -1, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd_psd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 8, 64, 64, KLA_PATH_AUTO, 0, nullptr) ==
        KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_fwd_psd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 0, 64, 64, KLA_PATH_AUTO, 0, nullptr) ==
        KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_fwd_noalloc(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 96,
                              64, 64, KLA_PATH_AUTO, 0, nullptr) == KLA_ERR_UNSUPPORTED);
  // a workspace beyond the static scratch buffer is refused before anything is enqueued
  CHECK(kla_chunk_fwd_noalloc(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 64, 8192, 16,
                              128, 128, 64, KLA_PATH_SEQUENTIAL, 0, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(std::strstr(kla_last_error(), "scratch") != nullptr);

  // backward
  CHECK(kla_chunk_bwd(KLA_DTYPE_F32, KLA_BETA_KACZMARZ, F, F, F, F, F, 1e-6f, nullptr, F, nullptr, F, F, F, F, F, nullptr,
                      1, 64, 1, 256, 64, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_chunk_bwd(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, 1e-6f, nullptr, nullptr, nullptr, F, F, F, F, F,
                      nullptr, 1, 64, 1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_bwd(KLA_DTYPE_F32, KLA_BETA_KACZMARZ, P, P, P, F, F, 1e-6f, nullptr, F, nullptr, F, F, F, F, F, MIS, 1, 64,
                      1, 64, 64, 64, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_chunk_bwd(KLA_DTYPE_F32, KLA_BETA_KACZMARZ, nullptr, nullptr, nullptr, nullptr, nullptr, 1e-6f, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 64, 64, 64,
                      nullptr) == KLA_OK);

  // decode
  CHECK(kla_decode_step(P, P, P, F, F, 1e-6f, F, F, -1, 2, 128, 128, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_decode_step(P, P, P, F, F, 1e-6f, F, F, 4, 2, 100, 128, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_decode_step(P, P, P, F, F, 1e-6f, nullptr, F, 4, 2, 128, 128, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, 1e-6f, nullptr, nullptr, 0, 2, 128, 128, nullptr) ==
        KLA_OK);
  CHECK(kla_decode_step_f32(F, F, F, F, F, 1e-6f, MIS, F, 4, 2, 128, 128, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_decode_step_ex(KLA_DTYPE_F32, static_cast<kla_beta_mode>(3), P, P, P, F, F, 1e-6f, F, F, 4, 2, 128, 128,
                           nullptr) == KLA_ERR_INVALID_ARG);

  // log-linear
  CHECK(kla_loglinear_decode_step(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, F, 1e-6f, F, F, 2, 2, 128, 128, 0, 0,
                                  nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_loglinear_decode_step(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, F, 1e-6f, F, F, 2, 2, 128, 128, 4, 8,
                                  nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_loglinear_decode_step(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, F, 1e-6f, F, F, 2, 2, 128, 128, 16,
                                  -1, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_loglinear_decode_step(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, MIS, 1e-6f, F, F, 2, 2, 128, 128, 16,
                                  5, nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_loglinear_decode_step(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  1e-6f, nullptr, nullptr, 0, 2, 128, 128, 31, (1 << 30) - 1, nullptr) == KLA_OK);
  CHECK(kla_loglinear_fwd(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, F, 1e-6f, F, 1, 129, 1, 64, 64, 8, 64,
                          nullptr) == KLA_ERR_INVALID_ARG);
  CHECK(kla_loglinear_fwd(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, P, P, P, F, F, nullptr, 1e-6f, F, 1, 64, 1, 64, 64, 8, 64,
                          nullptr) == KLA_ERR_INVALID_ARG);

  // planning: path choice and workspace sizes, host only
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int dk : {64, 128, 256})
      for (int dv : {64, 128})
        for (int T : {1, 63, 64, 65, 1000, 131072})
          for (int BH : {1, 3, 16, 128, 4096}) {
            if (dtype == 1 && dk == 256) continue;
            kla_path path;
            int segs = -1;
            size_t ws = 0;
            CHECK(kla_plan(static_cast<kla_dtype>(dtype), 1, T, BH, dk, dv, 64, KLA_PATH_AUTO, 0, 256, &path, &segs, &ws) ==
                  KLA_OK);
            const size_t nc = (T + 63) / 64;
            CHECK(segs >= 1 && static_cast<size_t>(segs) <= nc);
            CHECK(ws >= nc * BH * 13056);
            CHECK(path == KLA_PATH_SEQUENTIAL || path == KLA_PATH_SCAN);
          }
  CHECK(kla_plan(KLA_DTYPE_BF16, 1, 64, 1, 64, 64, 64, KLA_PATH_AUTO, 0, 256, nullptr, nullptr, nullptr) == KLA_OK);
  CHECK(kla_plan(KLA_DTYPE_BF16, 1, 64, 1, 64, 64, 64, static_cast<kla_path>(4), 0, 256, nullptr, nullptr, nullptr) ==
        KLA_ERR_INVALID_ARG);

  // timing hook: names, and a collect with nothing recorded
  char longname[64];
  std::memset(longname, 'k', sizeof longname - 1);
  longname[sizeof longname - 1] = 0;
  CHECK(kla_timing_select(longname) == KLA_ERR_INVALID_ARG);
  CHECK(kla_timing_select("kla_state_seq") == KLA_OK);
  CHECK(kla_timing_select(nullptr) == KLA_OK);
  CHECK(kla_timing_enable(1) == KLA_OK);
  CHECK(kla_chunk_fwd(P, P, P, F, F, 1e-6f, nullptr, F, nullptr, 1, 64, 1, 96, 64, 64, nullptr) == KLA_ERR_UNSUPPORTED);
  CHECK(kla_timing_enable(0) == KLA_OK);
  kla_kernel_timing rec[4];
  CHECK(kla_timing_collect(rec, 4) == 0);
  CHECK(kla_timing_collect(nullptr, 0) == 0);
  CHECK(std::strstr(kla_version(), "gfx950") != nullptr);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi checks passed\n");
  return 0;
}
