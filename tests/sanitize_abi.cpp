// Drives the host-side validation of every libringattn entry point with
// fake, never-dereferenced device addresses, for a build of the library's
// host code under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitize.py; the device code is compiled as usual).  Every call
// here is rejected before any HIP call, so no GPU is touched.  Prints "ok".
#include <cstdint>
#include <cstdio>

#include "libringattn.h"

namespace {

const uintptr_t kFake = 0x100000;  // 16-byte aligned, never dereferenced

ra_tensor T(int64_t b, int64_t s, int64_t h, int64_t d, int32_t dt = RA_BF16, uintptr_t data = kFake) {
  ra_tensor t{};
  t.data = (void*)data;
  t.dtype = dt;
  t.shape[0] = b; t.shape[1] = s; t.shape[2] = h; t.shape[3] = d;
  t.stride[3] = 1; t.stride[2] = d; t.stride[1] = h * d; t.stride[0] = s * h * d;
  return t;
}
ra_tensor R(int64_t b, int64_t h, int64_t s) {  // row statistics [B, H, S, 1]
  ra_tensor t{};
  t.data = (void*)kFake;
  t.dtype = RA_F32;
  t.shape[0] = b; t.shape[1] = h; t.shape[2] = s; t.shape[3] = 1;
  t.stride[0] = h * s; t.stride[1] = s; t.stride[2] = 1; t.stride[3] = 1;
  return t;
}

int g_fail = 0;
void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("%s: got %d, want %d (%s)\n", what, got, want, ra_last_error());
    g_fail = 1;
  }
}

}  // namespace

int main() {
  ra_tensor q = T(1, 512, 4, 128), k = T(1, 4096, 1, 128), o = T(1, 512, 4, 128);
  ra_tensor lse = R(1, 4, 512), bad_lse = R(1, 4, 511);
  ra_opts opts{};
  opts.o_out = &o;
  // ra_rank_share and its variants
  expect(ra_rank_share(&q, &k, &k, 8, 7, 1, nullptr), RA_E_NULL, "share without o_out");
  expect(ra_rank_share(&q, &k, &k, 0, 0, 1, &opts), RA_E_RANGE, "share P < 1");
  expect(ra_rank_share(&q, &k, &k, 8, 8, 1, &opts), RA_E_RANGE, "share rank >= P");
  ra_tensor k3 = T(1, 4095, 1, 128);
  expect(ra_rank_share(&q, &k3, &k3, 8, 7, 1, &opts), RA_E_SHAPE, "share N % P");
  opts.lse_out = &bad_lse;
  expect(ra_rank_share(&q, &k, &k, 8, 7, 1, &opts), RA_E_SHAPE, "share lse shape");
  opts.lse_out = &lse;
  ra_tensor qmis = T(1, 512, 4, 128, RA_BF16, kFake + 8);
  expect(ra_rank_share(&qmis, &k, &k, 8, 7, 1, &opts), RA_E_LAYOUT, "share misaligned q");
  ra_tensor q96 = T(1, 512, 4, 96), k96 = T(1, 4096, 1, 96), o96 = T(1, 512, 4, 96);
  ra_opts o96opts{};
  o96opts.o_out = &o96;
  expect(ra_rank_share(&q96, &k96, &k96, 8, 7, 1, &o96opts), RA_E_UNSUPPORTED, "share d = 96");
  expect(ra_rank_share_zigzag(&q, &k3, &k3, 8, 7, 1, &opts), RA_E_SHAPE, "zigzag N % 2P");
  expect(ra_rank_share_padded(&q, &k, &k, 8, 7, 1, 0, &opts), RA_E_RANGE, "padded n_valid 0");
  expect(ra_rank_share_padded(&q, &k, &k, 8, 7, 1, 5000, &opts), RA_E_RANGE, "padded n_valid > N");
  // ra_step, state kernels
  ra_tensor oacc = T(1, 512, 4, 128, RA_F32), m = R(1, 4, 512), l = R(1, 4, 512);
  ra_tensor kb = T(1, 512, 1, 128);
  expect(ra_step(&q, &kb, &kb, &oacc, &m, &l, -1, 0, 1, nullptr), RA_E_RANGE, "step negative offset");
  expect(ra_step(&q, &kb, &kb, &o, &m, &l, 0, 0, 1, nullptr), RA_E_DTYPE, "step bf16 state");
  expect(ra_step(&q, &kb, &kb, &oacc, &m, &bad_lse, 0, 0, 1, nullptr), RA_E_SHAPE, "step l shape");
  expect(ra_step(&q, &kb, &kb, &oacc, &m, &l, 0, 4096, 1, nullptr), RA_OK, "step SKIP (no launch)");
  expect(ra_state_init(&o, &m, &l, nullptr), RA_E_DTYPE, "init bf16 state");
  expect(ra_merge(&oacc, &m, &l, &o, &m, &l, nullptr), RA_E_DTYPE, "merge bf16 second state");
  expect(ra_merge(&oacc, &m, &l, &oacc, &m, &bad_lse, nullptr), RA_E_SHAPE, "merge l_b shape");
  ra_opts fopts{};
  fopts.lse_out = &lse;
  expect(ra_finalize(&oacc, &l, &fopts), RA_E_NULL, "finalize lse without m");
  ra_tensor big = T(1, int64_t(1) << 20, int64_t(1) << 10, 128, RA_F32);
  ra_tensor bigr = R(1, int64_t(1) << 10, int64_t(1) << 20);
  expect(ra_finalize(&big, &bigr, nullptr), RA_E_RANGE, "finalize beyond the work-item limit");
  // backward
  ra_tensor g = T(1, 512, 4, 128, RA_F32), gk = T(1, 4096, 1, 128, RA_F32), delta = R(1, 4, 512);
  expect(ra_rank_share_bwd(&q, &k, &k, &q, &lse, &q, 8, 7, 1, &g, &gk, &gk, nullptr, nullptr), RA_E_NULL,
         "backward without delta");
  expect(ra_rank_share_bwd(&q, &k, &k, &q, &lse, &q, 8, 7, 1, &o, &gk, &gk, &delta, nullptr), RA_E_DTYPE,
         "backward bf16 dq");
  expect(ra_rank_share_zigzag_bwd(&q, &k3, &k3, &q, &lse, &q, 8, 7, 1, &g, &gk, &gk, &delta, nullptr), RA_E_SHAPE,
         "zigzag backward N % 2P");
  expect(ra_rank_share_padded_bwd(&q, &k, &k, &q, &lse, &q, 8, 7, 1, 0, &g, &gk, &gk, &delta, nullptr), RA_E_RANGE,
         "padded backward n_valid 0");
  ra_tensor qb = T(1, 512, 2049, 128), gb = T(1, 512, 2049, 128, RA_F32);
  ra_tensor lb = R(1, 2049, 512);
  expect(ra_rank_share_bwd_noalloc(&qb, &k, &k, &qb, &lb, &qb, 8, 7, 1, &gb, &gk, &gk, nullptr), RA_E_RANGE,
         "no-alloc backward beyond its workspace");
  // host planner queries
  int8_t plan[64];
  expect((int)ra_plan_tiles(0, 100, 0, 100, 1, 32, 32, plan, 16), 16, "plan tiles (16 entries)");
  expect((int)ra_plan_tiles(0, 100, 0, 100, 1, 32, 32, plan, 15), RA_E_RANGE, "plan tiles, out too short");
  expect(ra_classify(0, 10, 20, 10, 1), 0, "classify SKIP");
  int64_t bm = 0, bn = 0;
  expect(ra_tile_shape(RA_BF16, 128, &bm, &bn), RA_OK, "tile shape");
  if (ra_flops(10, 10, 0, 0, 1, 64, 1) <= 0 || ra_share_flops(1, 64, 4, 3, 1, 64, 1) <= 0 ||
      ra_share_flops_zigzag(1, 64, 4, 3, 1, 64, 1) <= 0 || ra_ring_block(4, 1, 3) != 2) {
    std::printf("planner queries\n");
    g_fail = 1;
  }
  if (!g_fail) std::printf("ok\n");
  return g_fail;
}
