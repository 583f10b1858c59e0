// Host check of the causal decisions the kernels take, against the oracle's
// classifier (oracle/ra_oracle.c, linked in by tests/test_plan_native.py).
//
// The forward kernels (and the dQ kernel, which walks keys the same way)
// take three integer decisions per workgroup of BM = 256 query rows (waves of
// 32 or 64 rows, in row blocks of 32) and key block [k0, k0 + nk):
//   1. how many 64-key tiles to walk: ra_plan_key_tiles;
//   2. per tile and wave, whether the softmax needs its masked form:
//      ra_plan_tile_masked on the tile's position relative to the wave's first
//      query (32-bit, saturated at -2^30 as the kernel's tile cursor keeps it),
//      then per 32-key unit (ra_plan_half_valid keys) and row block the same
//      test again;
//   3. per masked unit and query row, the visible keys: a prefix of
//      ra_plan_visible_prefix keys.
// The dK/dV kernel starts its walk over query tiles of 128 rows at
// ra_plan_first_query_tile (checked for tiles of 64 rows too), and skips the
// per-element test of the 32-query units of a tile from
// ra_plan_first_full_unit on, which must be exactly the units whose every
// pair with the wave's 32 keys is visible, all keys before the key end.
// Every decision must agree bit for bit with
// orc_classify / orc_visible_pairs: a tile is walked iff it holds a visible
// pair; a tile or unit skips the mask only when every pair is visible; the
// visible prefix counts exactly the visible keys; the query tiles before the
// first one see none of the workgroup's keys.  Prints "ok" or the first
// disagreement.
#include "ra_plan.h"

#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
int orc_classify(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal);
int64_t orc_visible_pairs(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal);
}

namespace {

constexpr int BM = 256, BN = 64, UNIT = 32;
long long g_checked = 0;

bool fail(const char* what, long long q0, long long nq, long long k0, long long nk, int causal, long long a,
          long long b) {
  std::printf("%s: q0 %lld nq %lld k0 %lld nk %lld causal %d: kernel %lld oracle %lld\n", what, q0, nq, k0, nk,
              causal, a, b);
  return false;
}

// One forward workgroup (rows [q0, q0 + nq), nq <= BM) against one key
// block; waves of wave_rows rows, each in row blocks of 32 (the 32- and the
// 64-rows-per-wave kernels: the tile flag is taken for the wave's first
// row, the unit tests per row block).
bool check_forward(int64_t q0, int nq, int64_t k0, int64_t nk, int causal, int wave_rows) {
  const int64_t n = ra_plan_key_tiles(q0, nq, k0, nk, causal, BN);
  const int64_t all = (nk + BN - 1) / BN;
  for (int64_t t = 0; t < all; ++t) {
    const int64_t kt = k0 + t * BN, nvt = nk - t * BN < BN ? nk - t * BN : BN;
    const bool walked = t < n;
    const bool visible = orc_classify(q0, nq, kt, nvt, causal) != 0;
    ++g_checked;
    if (walked != visible) return fail("tile walked iff it holds a visible pair", q0, nq, k0, nk, causal, walked, visible);
  }
  for (int w = 0; w * wave_rows < nq; ++w) {
    const int64_t q0w = q0 + w * wave_rows;
    const int nqw = nq - w * wave_rows < wave_rows ? nq - w * wave_rows : wave_rows;
    // the kernel's cursor: relative position of the block saturated at
    // +-2^30, then advanced by BN per tile
    const int64_t rel0 = k0 - q0w;
    const int sat = 1 << 30;
    const int crel0 = rel0 < -sat ? -sat : (rel0 > sat ? sat : (int)rel0);
    for (int64_t t = 0; t < n; ++t) {
      const int64_t kt = k0 + t * BN;
      const int nvt = (int)(nk - t * BN < BN ? nk - t * BN : BN);
      const bool flag = ra_plan_tile_masked<int>(crel0 + (int)t * BN, nvt, BN, causal);
      const bool want = nvt < BN || orc_classify(q0w, nqw, kt, nvt, causal) != 1;
      ++g_checked;
      if (flag != want) return fail("tile mask flag iff ragged or not FULL for the wave", q0w, nqw, kt, nvt, causal, flag, want);
      int64_t tile_pairs = 0;  // visible pairs of the wave's rows over both units, as the kernel counts them
      for (int hf = 0; hf < 2; ++hf) {
        const int nvu = ra_plan_half_valid(nvt, hf, UNIT);
        const int64_t ku = kt + hf * UNIT;
        for (int rb = 0; rb * 32 < nqw; ++rb) {
          const int64_t q0r = q0w + 32 * rb;
          const int nqr = nqw - 32 * rb < 32 ? nqw - 32 * rb : 32;
          const bool masked = flag && ra_plan_tile_masked<int64_t>(ku - q0r, nvu, UNIT, causal);
          if (!masked) {
            // the plain softmax: every one of the unit's 32 slots holds a key
            // visible to every row of the row block
            const int64_t vis = orc_visible_pairs(q0r, nqr, ku, nvu, causal);
            ++g_checked;
            if (nvu != UNIT || vis != (int64_t)nqr * UNIT)
              return fail("unmasked unit has every pair visible", q0r, nqr, ku, nvu, causal, (long long)nqr * UNIT,
                          vis);
            tile_pairs += (int64_t)nqr * UNIT;
            continue;
          }
          for (int i = 0; i < nqr; ++i) {
            const int64_t lim = ra_plan_visible_prefix(q0r + i, ku, nvu, causal);
            const int64_t vis_all = orc_visible_pairs(q0r + i, 1, ku, nvu, causal);
            const int64_t vis_pre = orc_visible_pairs(q0r + i, 1, ku, lim, causal);
            ++g_checked;
            if (lim != vis_all || vis_pre != lim)
              return fail("visible prefix is exactly the visible keys", q0r + i, 1, ku, nvu, causal, lim, vis_all);
            tile_pairs += lim;
          }
        }
      }
      // the two units cover exactly the tile's keys
      const int64_t want_pairs = orc_visible_pairs(q0w, nqw, kt, nvt, causal);
      ++g_checked;
      if (tile_pairs != want_pairs)
        return fail("units cover the tile's visible pairs", q0w, nqw, kt, nvt, causal, tile_pairs, want_pairs);
    }
  }
  return true;
}

// The dK/dV walk of a workgroup of keys [kfirst, kfirst + nk) over a query
// chunk of nqc rows from position qpos, in tiles of qt rows.
bool check_first_query_tile(int64_t kfirst, int64_t nk, int64_t qpos, int nqc, int causal, int qt) {
  const int ntq = (nqc + qt - 1) / qt;
  const int t0 = ra_plan_first_query_tile(kfirst, qpos, nqc, qt, causal);
  for (int t = 0; t < ntq; ++t) {
    const int rows = nqc - t * qt < qt ? nqc - t * qt : qt;
    const int64_t vis = orc_visible_pairs(qpos + (int64_t)t * qt, rows, kfirst, nk, causal);
    ++g_checked;
    if ((t >= t0) != (vis > 0))
      return fail("query tile walked iff it sees a key of the workgroup", qpos + (int64_t)t * qt, rows, kfirst, nk,
                  causal, t >= t0, vis);
  }
  return true;
}

// The dK/dV kernel's per-tile split: the wave's keys klast - 31 .. klast
// (those before kv_end live), a tile of nu units of 32 queries from q0.
bool check_first_full_unit(int64_t klast, int64_t kv_end, int64_t q0, int nu, int causal) {
  const int first = ra_plan_first_full_unit(klast, kv_end, q0, nu, causal);
  for (int v = 0; v < nu; ++v) {
    const int64_t q0u = q0 + 32 * v;
    const bool want = klast < kv_end && orc_visible_pairs(q0u, 32, klast - 31, 32, causal) == 32 * 32;
    ++g_checked;
    if ((v >= first) != want)
      return fail("unit skips the test iff every key is live and sees every query", q0u, 32, klast - 31, 32, causal,
                  v >= first, want);
  }
  return true;
}

}  // namespace

int main() {
  // structured sweep around the tile and wave boundaries
  const int nqs[] = {1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256};
  const int64_t nks[] = {1, 2, 31, 32, 33, 63, 64, 65, 100, 128, 129, 255, 256, 300, 513};
  const int64_t q0s[] = {0, 1, 31, 32, 100, 255, 256, 1000, 4096};
  const int64_t dks[] = {-600, -513, -300, -256, -129, -128, -65, -64, -63, -33, -32, -31, -1, 0,
                         1, 31, 32, 33, 63, 64, 65, 100, 200, 255, 256, 257};
  for (int causal = 0; causal < 2; ++causal)
    for (int64_t q0 : q0s)
      for (int nq : nqs)
        for (int64_t dk : dks)
          for (int64_t nk : nks) {
            const int64_t k0 = q0 + dk;
            if (k0 < 0) continue;
            for (int wr : {32, 64})
              if (!check_forward(q0, nq, k0, nk, causal, wr)) return 1;
          }
  // random positions, including a block far before the queries (the
  // saturated relative position) and long blocks
  std::mt19937_64 rng(20261203);
  for (int it = 0; it < 20000; ++it) {
    const int causal = (int)(rng() & 1);
    const int nq = 1 + (int)(rng() % BM);
    const int64_t q0 = (it % 50 == 0) ? (int64_t(3) << 30) + (int64_t)(rng() % 1000) : (int64_t)(rng() % 20000);
    const int64_t nk = 1 + (int64_t)(rng() % 2000);
    const int64_t k0 = (it % 50 == 0) ? (int64_t)(rng() % 1000) : (int64_t)(rng() % 22000);
    for (int wr : {32, 64})
      if (!check_forward(q0, nq, k0, nk, causal, wr)) return 1;
  }
  for (int causal = 0; causal < 2; ++causal)
    for (int64_t qpos : {0, 64, 100, 1000})
      for (int nqc : {1, 63, 64, 65, 127, 128, 129, 200, 256, 257, 512})
        for (int64_t dk = -300; dk <= 900; dk += 7)
          for (int64_t nk : {1, 64, 127, 128})
            for (int qt : {64, 128}) {
              const int64_t kfirst = qpos + dk;
              if (kfirst < 0) continue;
              if (!check_first_query_tile(kfirst, nk, qpos, nqc, causal, qt)) return 1;
            }
  const int64_t q0us[] = {0, 31, 32, 100, 4096, (int64_t(3) << 30) + 7};
  for (int causal = 0; causal < 2; ++causal)
    for (int64_t q0u : q0us)
      for (int64_t dk = -70; dk <= 170; ++dk)
        for (int64_t de = -34; de <= 34; ++de) {
          const int64_t klast = q0u + dk;
          if (klast < 31) continue;
          for (int nu : {1, 2, 4})
            if (!check_first_full_unit(klast, klast + de, q0u, nu, causal)) return 1;
        }
  std::printf("ok %lld\n", g_checked);
  return 0;
}
