/*
 * Host-side checks of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer, against the library built with both on its host
 * code. It runs with no GPU visible and refuses to run otherwise: a call that
 * passes validation reaches its launch code and fails with HA_ERR_DEVICE
 * instead of running a kernel, so every argument check, size query, workspace
 * layout and grid computation runs on the CPU. Pointers are never dereferenced
 * by the library; the ones passed here are plain numbers.
 *
 * Exit status 0 and the line "abi sanitizer driver: N calls, all checks
 * passed" mean no sanitizer report and every expected status matched.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "hybrid_attn.h"

static long long g_calls = 0;
static int g_fail = 0;

static void expect(const char* what, int got, int want) {
  ++g_calls;
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    g_fail = 1;
  }
}

/* A status a call with no device may return: anything but success. */
static void expect_error(const char* what, int got) {
  ++g_calls;
  if (got <= HA_OK || got > HA_ERR_NONFINITE) {
    fprintf(stderr, "FAIL %s: status %d is not an error code\n", what, got);
    g_fail = 1;
  }
}

#define P(x) ((void*)(uintptr_t)(x))
#define GiB(x) ((uintptr_t)(x) << 30)

/* Buffers 64 GiB apart: no two overlap unless a case moves one. */
static uintptr_t buf(int i) { return GiB(64) * (uintptr_t)(i + 1); }

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* xorshift64* */
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 0x2545F4914F6CDD1Dull;
}

static int pick_int(void) {
  static const int v[] = {-7, -1, 0, 1, 2, 3, 12, 17, 21, 32, 40, 64, 100, 128, 129, 256, 1560, 3600,
                          32760, 75600, 1 << 20, INT_MAX / 2, INT_MAX - 1, INT_MAX, INT_MIN};
  return v[next_u64() % (sizeof v / sizeof v[0])];
}

static void* pick_ptr(int i) {
  switch (next_u64() % 6) {
    case 0: return NULL;
    case 1: return P(buf(i) + 4);          /* misaligned for 16 */
    case 2: return P(buf(0));              /* may overlap buffer 0 */
    default: return P(buf(i));
  }
}

int hipGetDeviceCount(int* count); /* from the HIP runtime the library links */

int main(void) {
  char name[128];
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == 0 && ndev > 0) {
    fprintf(stderr, "abi sanitizer driver: %d GPU(s) visible; it only runs with none "
                    "(HIP_VISIBLE_DEVICES=-1 ROCR_VISIBLE_DEVICES=-1)\n", ndev);
    return 2;
  }

  /* version and status strings for every int that could reach them */
  if (hybrid_attn_version() < 100) g_fail = 1;
  for (int s = -3; s <= 12; ++s)
    if (!hybrid_attn_status_string((ha_status)s)[0]) g_fail = 1;

  /* size queries over a grid of shapes, including overflowing ones */
  for (int i = 0; i < 20000; ++i) {
    const int B = pick_int(), H = pick_int(), T = pick_int(), L = pick_int(), d = pick_int();
    (void)hybrid_attn_workspace_bytes(B, H, T, L, d, (int)(next_u64() & 1));
    (void)hybrid_attn_state_workspace_bytes(B, H, T, L, d);
    (void)hybrid_attn_fmap_workspace_bytes(B, H, T, L, d, (int)(next_u64() & 1));
    (void)hybrid_attn_gated_workspace_bytes(B, H, T, L, d, (int)(next_u64() & 1));
    (void)hybrid_attn_gates_workspace_bytes(B, H, T, L);
    (void)hybrid_attn_kvcache_workspace_bytes(B, H, T, L, d, pick_int());
    (void)hybrid_attn_token_level_workspace_bytes(B, H, T, L, d);
    g_calls += 7;
  }
  /* the documented sizes */
  {
    const size_t up = 256;
#define UP(x) (((x) + up - 1) / up * up)
    const size_t gram = (size_t)12 * 21 * 128 * 256 * 4, snaps = (size_t)12 * 21 * 128 * 128 * 4;
    expect("480p workspace", hybrid_attn_workspace_bytes(1, 12, 21 * 1560, 1560, 128, 1) == UP(gram) + UP(snaps), 1);
    expect("denoise workspace", (int)hybrid_attn_workspace_bytes(1, 12, 1560, 1560, 128, 0), 0);
    expect("noalloc scratch", hybrid_attn_noalloc_scratch_bytes() == ((size_t)64 << 20), 1);
#undef UP
  }

  /* forward: one valid call (reaches the launches, which fail without device
     code) and each validation rule */
  const int B = 1, H = 2, T = 256, L = 128, d = 128;
  const size_t ws = hybrid_attn_workspace_bytes(B, H, T, L, d, 1);
#define FWD(q_, st_, out_, ws_, wsb_, T_, L_, d_, upd_)                                                        \
  hybrid_attn_forward(P(q_), P(buf(1)), P(buf(2)), P(buf(3)), P(buf(4)), P(buf(5)), (const float*)P(buf(6)), \
                      (const float*)P(buf(7)), (float*)P(st_), P(out_), P(ws_), wsb_, B, H, T_, d_, L_, HA_BF16, \
                      upd_, 0.0f, NULL)
  expect("forward valid (no device)", FWD(buf(0), buf(8), buf(9), buf(10), ws, T, L, d, 1), HA_ERR_DEVICE);
  expect("forward denoise valid (no device)", FWD(buf(0), buf(8), buf(9), 0, 0, T, L, d, 0), HA_ERR_DEVICE);
  expect("forward null q", FWD(0, buf(8), buf(9), buf(10), ws, T, L, d, 1), HA_ERR_NULL);
  expect("forward T % L", FWD(buf(0), buf(8), buf(9), buf(10), ws, T + 1, L, d, 1), HA_ERR_SHAPE);
  expect("forward d", FWD(buf(0), buf(8), buf(9), buf(10), ws, T, L, 96, 1), HA_ERR_UNSUPPORTED);
  expect("forward align", FWD(buf(0) + 8, buf(8), buf(9), buf(10), ws, T, L, d, 1), HA_ERR_ALIGN);
  expect("forward workspace", FWD(buf(0), buf(8), buf(9), buf(10), ws - 1, T, L, d, 1), HA_ERR_WORKSPACE);
  expect("forward alias ws/q", FWD(buf(0), buf(8), buf(9), buf(0), ws, T, L, d, 1), HA_ERR_ALIAS);
  expect("forward alias out/state", FWD(buf(0), buf(8), buf(8), buf(10), ws, T, L, d, 1), HA_ERR_ALIAS);
#undef FWD
#define MIXF(mix_, out_, dt_)                                                                                  \
  hybrid_attn_forward_mix(P(buf(0)), P(buf(1)), P(buf(2)), P(buf(3)), P(buf(4)), P(buf(5)),                     \
                          (const float*)P(buf(6)), (const float*)P(buf(7)), (float*)P(buf(8)), P(out_),         \
                          (const float*)P(mix_), P(buf(10)), ws, B, H, T, d, L, dt_, 1, 0.0f, NULL)
  expect("mix valid (no device)", MIXF(buf(11), buf(9), HA_BF16), HA_ERR_DEVICE);
  expect("mix null weights", MIXF(0, buf(9), HA_BF16), HA_ERR_NULL);
  expect("mix misaligned weights", MIXF(buf(11) + 4, buf(9), HA_BF16), HA_ERR_ALIGN);
  expect("mix fp32", MIXF(buf(11), buf(9), HA_FP32), HA_ERR_UNSUPPORTED);
  expect("mix alias out/weights", MIXF(buf(11), buf(11), HA_BF16), HA_ERR_ALIAS);
#undef MIXF
  expect("noalloc too large",
         hybrid_attn_forward_noalloc(P(buf(0)), P(buf(1)), P(buf(2)), P(buf(3)), P(buf(4)), P(buf(5)),
                                     (const float*)P(buf(6)), (const float*)P(buf(7)), (float*)P(buf(8)), P(buf(9)),
                                     1, 40, 21 * 3600, 128, 3600, HA_BF16, 1, 0.0f, NULL),
         HA_ERR_SCRATCH);
  expect("noalloc valid (no device)",
               hybrid_attn_forward_noalloc(P(buf(0)), P(buf(1)), P(buf(2)), P(buf(3)), P(buf(4)), P(buf(5)),
                                           (const float*)P(buf(6)), (const float*)P(buf(7)), (float*)P(buf(8)),
                                           P(buf(9)), B, H, T, d, L, HA_BF16, 1, 0.0f, NULL),
         HA_ERR_DEVICE);

  /* every entry point with random arguments: an error code, never a crash or
     a sanitizer report */
  for (int it = 0; it < 4000; ++it) {
    const int b = pick_int() % 9, h = pick_int() % 50, t = pick_int(), l = pick_int(), dd = (int)(next_u64() & 1) ? 64 : 128;
    const int upd = (int)(next_u64() & 1), dt = (int)(next_u64() % 3);
    const size_t wsb = (size_t)(next_u64() % (1ull << 40));
    snprintf(name, sizeof name, "random call %d", it);
    expect_error(name, hybrid_attn_forward(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3), pick_ptr(4),
                                           pick_ptr(5), (const float*)pick_ptr(6), (const float*)pick_ptr(7),
                                           (float*)pick_ptr(8), pick_ptr(9), pick_ptr(10), wsb, b, h, t, dd, l,
                                           (ha_dtype)dt, upd, 0.0f, NULL));
    expect_error(name, hybrid_attn_intra_readout(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3),
                                                 (const float*)pick_ptr(4), (long long)pick_int() * 4,
                                                 (long long)pick_int() * 4, pick_ptr(9), b, h, t, dd, l,
                                                 (ha_dtype)dt, 0.0f, NULL));
    expect_error(name, hybrid_attn_state_update(pick_ptr(4), pick_ptr(5), (const float*)pick_ptr(6),
                                                (const float*)pick_ptr(7), (float*)pick_ptr(8),
                                                (float*)pick_ptr(11), pick_ptr(10), wsb, b, h, t, dd, l,
                                                (ha_dtype)dt, NULL));
    expect_error(name, hybrid_attn_forward_fmap(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3), pick_ptr(4),
                                                pick_ptr(5), (const float*)pick_ptr(6), (const float*)pick_ptr(7),
                                                (float*)pick_ptr(8), pick_ptr(9), pick_ptr(10), wsb, b, h, t, dd, l,
                                                (ha_dtype)dt, upd, 0.0f, NULL));
    expect_error(name, hybrid_attn_forward_gated(pick_ptr(11), pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3),
                                                 pick_ptr(4), pick_ptr(5), pick_ptr(12), (const float*)pick_ptr(13),
                                                 (float*)pick_ptr(8), pick_ptr(9), pick_ptr(10), wsb, b, h, t, dd,
                                                 pick_int(), l, (ha_dtype)dt, upd, (int)(next_u64() & 1), 0.0f,
                                                 NULL));
    expect_error(name, hybrid_attn_gates(pick_ptr(11), pick_ptr(12), (const float*)pick_ptr(13),
                                         (float*)pick_ptr(6), (float*)pick_ptr(7), pick_ptr(10), wsb, b, h, t,
                                         pick_int(), l, (ha_dtype)dt, NULL));
    expect_error(name, hybrid_attn_kvcache_forward(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(14),
                                                   pick_ptr(15), pick_ptr(9), pick_ptr(10), wsb, b, h, t, dd, l,
                                                   pick_int(), pick_int(), (ha_dtype)dt, 0.0f, NULL));
    expect_error(name, hybrid_attn_forward_token_level(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3),
                                                       pick_ptr(4), pick_ptr(5), (const float*)pick_ptr(6),
                                                       (const float*)pick_ptr(7), (float*)pick_ptr(8),
                                                       pick_ptr(9), pick_ptr(10), wsb, b, h, t, dd, l,
                                                       (ha_dtype)dt, upd, 0.0f, NULL));
    expect_error(name, hybrid_attn_forward_mix(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3), pick_ptr(4),
                                               pick_ptr(5), (const float*)pick_ptr(6), (const float*)pick_ptr(7),
                                               (float*)pick_ptr(8), pick_ptr(9), (const float*)pick_ptr(11),
                                               pick_ptr(10), wsb, b, h, t, dd, l, (ha_dtype)dt, upd, 0.0f, NULL));
    expect_error(name, hybrid_attn_forward_noalloc(pick_ptr(0), pick_ptr(1), pick_ptr(2), pick_ptr(3),
                                                   pick_ptr(4), pick_ptr(5), (const float*)pick_ptr(6),
                                                   (const float*)pick_ptr(7), (float*)pick_ptr(8), pick_ptr(9), b,
                                                   h, t, dd, l, (ha_dtype)dt, upd, 0.0f, NULL));
  }
  if (g_fail) return 1;
  printf("abi sanitizer driver: %lld calls, all checks passed\n", g_calls);
  return 0;
}
