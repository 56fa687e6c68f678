// Host-side driver of the C ABI for an AddressSanitizer build of the library's host code.
//
// Every call below either is host-only (sizes, offsets, error strings) or fails one validation
// rule before any HIP call, so the program needs no GPU and launches nothing. Output arrays are
// heap-allocated with exactly the documented number of entries, so a write past the end of one is
// reported by the sanitizer. Exit status 0 means every expectation held; the test that builds and
// runs this program also requires the sanitizer to have reported nothing.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "flashgau.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// Fake, well-separated device addresses: never dereferenced, every call fails validation.
static void* fake(int slot, size_t delta = 0) {
  return reinterpret_cast<void*>((uintptr_t(1) << 40) + (uintptr_t(slot) << 30) + delta);
}

int main() {
  struct Shape { int64_t B, n, d, e, s, c; int causal; flashgau_dtype dt; };
  const Shape shapes[] = {{8, 4096, 768, 1536, 128, 256, 1, FLASHGAU_BF16},
                          {1, 512, 256, 512, 128, 128, 0, FLASHGAU_F32},
                          {3, 72, 200, 136, 24, 24, 1, FLASHGAU_BF16},
                          {2, 8192, 768, 1536, 128, 512, 0, FLASHGAU_BF16},
                          {0, 256, 64, 128, 128, 64, 1, FLASHGAU_BF16}};
  for (const Shape& sh : shapes) {
    size_t ws = 0, bws = 0;
    EXPECT(flashgau_workspace_size(sh.B, sh.n, sh.d, sh.e, sh.s, sh.c, sh.causal, sh.dt, &ws) ==
           FLASHGAU_OK);
    EXPECT(flashgau_workspace_bytes(sh.B, sh.n, sh.d, sh.e, sh.s, sh.c, sh.causal, sh.dt) == ws);
    EXPECT(flashgau_backward_workspace_size(sh.B, sh.n, sh.d, sh.e, sh.s, sh.c, sh.causal, sh.dt,
                                            &bws) == FLASHGAU_OK);
    EXPECT(bws >= ws);
    size_t* off = new size_t[FLASHGAU_WS_COUNT];
    EXPECT(flashgau_workspace_offsets(sh.B, sh.n, sh.d, sh.e, sh.s, sh.c, sh.causal, sh.dt, off) ==
           FLASHGAU_OK);
    for (int i = 1; i < FLASHGAU_WS_COUNT; ++i) EXPECT(off[i] >= off[i - 1] && off[i] % 256 == 0);
    delete[] off;
    int64_t ng = -1;
    EXPECT(flashgau_state_groups(sh.B, sh.n, sh.d, sh.e, sh.s, sh.c, sh.causal, sh.dt, &ng) ==
           FLASHGAU_OK);
    EXPECT(ng >= 1);
    size_t pk = 0;
    EXPECT(flashgau_packed_weights_size(sh.d, sh.e, sh.s, sh.dt, &pk) == FLASHGAU_OK && pk > 0);
    size_t ds = 0;
    EXPECT(flashgau_decode_state_size(sh.B, sh.d, sh.e, sh.s, sh.c, sh.dt, &ds) == FLASHGAU_OK);
    size_t* doff = new size_t[FLASHGAU_DS_COUNT];
    EXPECT(flashgau_decode_state_offsets(sh.B, sh.d, sh.e, sh.s, sh.c, sh.dt, doff) == FLASHGAU_OK);
    delete[] doff;
  }

  // invalid shapes: every size query reports the error and leaves its output alone
  size_t untouched = 12345;
  EXPECT(flashgau_workspace_size(2, 100, 64, 128, 128, 64, 1, FLASHGAU_BF16, &untouched) ==
         FLASHGAU_ERR_BAD_SHAPE);
  EXPECT(untouched == 12345);
  EXPECT(flashgau_workspace_size(1, int64_t(1) << 31, 64, 128, 128, 64, 1, FLASHGAU_BF16,
                                 &untouched) == FLASHGAU_ERR_BAD_SHAPE);
  EXPECT(flashgau_workspace_size(1, 128, 60, 128, 128, 64, 1, FLASHGAU_BF16, &untouched) ==
         FLASHGAU_ERR_UNSUPPORTED);
  EXPECT(flashgau_workspace_size(INT64_MAX / 2, 1 << 20, 8, 8, 8, 8, 1, FLASHGAU_BF16, &untouched) ==
         FLASHGAU_ERR_BAD_SHAPE);
  EXPECT(flashgau_workspace_size(1, 128, 64, 128, 128, 64, 1, (flashgau_dtype)7, &untouched) ==
         FLASHGAU_ERR_UNSUPPORTED);
  EXPECT(flashgau_workspace_bytes(1, 131072, 64, 128, 128, 131072, 1, FLASHGAU_BF16) == 0);
  EXPECT(flashgau_workspace_size(1, 128, 64, 128, 128, 64, 1, FLASHGAU_BF16, nullptr) ==
         FLASHGAU_ERR_NULL_PTR);

  // forward: one failing rule per call
  const int64_t B = 1, n = 128, d = 64, e = 128, s = 128, c = 64;
  size_t ws = 0;
  flashgau_workspace_size(B, n, d, e, s, c, 1, FLASHGAU_BF16, &ws);
  auto fwd = [&](void* X, void* O, void* W, size_t wsb, void* gamma) {
    return flash_gau_forward(X, fake(1), fake(2), fake(3), (const float*)gamma, (const float*)fake(5),
                             fake(6), c, 1, B, n, d, e, s, FLASHGAU_BF16, O, W, wsb, nullptr);
  };
  EXPECT(fwd(nullptr, fake(7), fake(8), ws, fake(4)) == FLASHGAU_ERR_NULL_PTR);
  EXPECT(fwd(fake(0, 8), fake(7), fake(8), ws, fake(4)) == FLASHGAU_ERR_MISALIGNED);
  EXPECT(fwd(fake(0), fake(7), fake(8), 1024, fake(4)) == FLASHGAU_ERR_WORKSPACE);
  EXPECT(fwd(fake(0), fake(0), fake(8), ws, fake(4)) == FLASHGAU_ERR_ALIASING);
  EXPECT(fwd(fake(0), fake(7), fake(7, 256), ws, fake(4)) == FLASHGAU_ERR_ALIASING);
  EXPECT(fwd(fake(0), fake(7), fake(8), ws, fake(4, 2)) == FLASHGAU_ERR_MISALIGNED);
  EXPECT(flash_gau_forward_rope(fake(0), fake(1), fake(2), fake(3), (const float*)fake(4),
                                (const float*)fake(5), fake(6), c, 1, -1.0f, B, n, d, e, s,
                                FLASHGAU_BF16, fake(7), fake(8), ws, nullptr) == FLASHGAU_ERR_BAD_SHAPE);
  void* events[2 * FLASHGAU_NUM_STAGES] = {};
  EXPECT(flash_gau_forward_timed(fake(0), fake(1), fake(2), fake(3), (const float*)fake(4),
                                 (const float*)fake(5), fake(6), c, 1, B, n, d, e, s, FLASHGAU_BF16,
                                 fake(7), fake(8), ws, nullptr, events,
                                 FLASHGAU_NUM_STAGES + 1) == FLASHGAU_ERR_NULL_PTR);
  // the per-kernel form (a start and a stop event per stage) is checked the same way; any other
  // count is rejected before an event is looked at
  EXPECT(flash_gau_forward_timed(fake(0), fake(1), fake(2), fake(3), (const float*)fake(4),
                                 (const float*)fake(5), fake(6), c, 1, B, n, d, e, s, FLASHGAU_BF16,
                                 fake(7), fake(8), ws, nullptr, events,
                                 2 * FLASHGAU_NUM_STAGES) == FLASHGAU_ERR_NULL_PTR);
  EXPECT(flash_gau_forward_timed(fake(0), fake(1), fake(2), fake(3), (const float*)fake(4),
                                 (const float*)fake(5), fake(6), c, 1, B, n, d, e, s, FLASHGAU_BF16,
                                 fake(7), fake(8), ws, nullptr, events,
                                 FLASHGAU_NUM_STAGES) == FLASHGAU_ERR_BAD_SHAPE);
  size_t pk = 0;
  flashgau_packed_weights_size(d, e, s, FLASHGAU_BF16, &pk);
  EXPECT(flash_gau_forward_packed(fake(0), fake(1), pk - 1, (const float*)fake(4),
                                  (const float*)fake(5), c, 1, B, n, d, e, s, FLASHGAU_BF16, fake(7),
                                  fake(8), ws, nullptr) == FLASHGAU_ERR_WORKSPACE);
  EXPECT(flash_gau_forward_packed(fake(0), fake(8, 512), pk, (const float*)fake(4),
                                  (const float*)fake(5), c, 1, B, n, d, e, s, FLASHGAU_BF16, fake(7),
                                  fake(8), ws, nullptr) == FLASHGAU_ERR_ALIASING);
  EXPECT(flash_gau_forward_noalloc(fake(0), fake(1), fake(2), fake(3), (const float*)fake(4),
                                   (const float*)fake(5), fake(6), 256, 1, 8, 4096, 768, 1536, 128,
                                   FLASHGAU_BF16, fake(7), nullptr) == FLASHGAU_ERR_TOO_LARGE);
  EXPECT(flash_gau_forward_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 64,
                                   1, 0, 256, 64, 128, 128, FLASHGAU_BF16, nullptr, nullptr) ==
         FLASHGAU_OK);

  // decode
  size_t st = 0;
  const int64_t DB = 2, Dd = 64, De = 96, Ds = 24, Dc = 8;
  flashgau_decode_state_size(DB, Dd, De, Ds, Dc, FLASHGAU_BF16, &st);
  flashgau_packed_weights_size(Dd, De, Ds, FLASHGAU_BF16, &pk);
  EXPECT(flash_gau_decode_step(fake(0), fake(1), pk, (const float*)fake(2), (const float*)fake(3), Dc,
                               16, 16, 0.0f, DB, Dd, De, Ds, FLASHGAU_BF16, fake(4), fake(5), st,
                               nullptr) == FLASHGAU_ERR_BAD_SHAPE);
  EXPECT(flash_gau_decode_step(fake(0), fake(1), pk, (const float*)fake(2), (const float*)fake(3), Dc,
                               3, 16, 0.0f, DB, Dd, De, Ds, FLASHGAU_BF16, fake(4), fake(5), 256,
                               nullptr) == FLASHGAU_ERR_WORKSPACE);

  // backward
  size_t bws = 0;
  flashgau_backward_workspace_size(B, n, d, e, s, c, 1, FLASHGAU_BF16, &bws);
  std::vector<void*> p(16);
  for (int i = 0; i < 16; ++i) p[i] = fake(i);
  EXPECT(flash_gau_backward(p[0], p[1], p[2], p[3], (const float*)p[4], (const float*)p[5], p[6], p[7],
                            c, 1, 0.0f, B, n, d, e, s, FLASHGAU_BF16, p[8], p[9], p[10], p[11],
                            (float*)p[12], (float*)p[13], p[14], p[15], 4096, nullptr) ==
         FLASHGAU_ERR_WORKSPACE);
  EXPECT(flash_gau_backward_saved(p[0], p[1], p[2], p[3], (const float*)p[4], (const float*)p[5], p[6],
                                  p[7], c, 1, 0.0f, B, n, d, e, s, FLASHGAU_BF16, p[0], p[9], p[10],
                                  p[11], (float*)p[12], (float*)p[13], p[14], p[15], bws, nullptr) ==
         FLASHGAU_ERR_ALIASING);
  EXPECT(flash_gau_forward_train(p[0], p[1], p[2], p[3], (const float*)p[4], (const float*)p[5], p[6],
                                 c, 1, 0.0f, B, n, d, e, s, FLASHGAU_BF16, p[7], p[8], ws, nullptr) ==
         FLASHGAU_ERR_WORKSPACE);

  // error strings: static text for every code, "unknown error" otherwise
  for (int code = -8; code <= 0; ++code) {
    const char* t = flashgau_strerror(code);
    EXPECT(t && strlen(t) > 0 && strcmp(t, "unknown error") != 0);
  }
  EXPECT(strcmp(flashgau_strerror(-99), "unknown error") == 0);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi driver: all host-side expectations held\n");
  return 0;
}
