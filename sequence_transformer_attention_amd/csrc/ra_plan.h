// ra_plan.h -- ring order and causal block/tile classes, shared by the host
// planner and the gfx950 kernels so both take bit-identical decisions.
//
// Ring order: glossary page "sequence parallelism transformers", section
// "Ring Attention", item "Ring Communication" (rank i sends to i+1 and
// receives from i-1; after s steps rank r holds the block of rank r - s).
// Classes: a key at global position kv is visible to a query at global
// position q iff !causal || kv <= q.  A (query range, key range) pair is SKIP
// when no pair is visible, FULL when all are, PARTIAL otherwise.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define RA_HD __host__ __device__ inline
#else
#define RA_HD inline
#endif

enum { RA_CLASS_SKIP = 0, RA_CLASS_FULL = 1, RA_CLASS_PARTIAL = 2 };

RA_HD int64_t ra_plan_ring_block(int64_t P, int64_t rank, int64_t s) {
  int64_t j = (rank - s) % P;
  return j < 0 ? j + P : j;
}

// 32-bit form for device loops (P, rank, s < 2^31).
RA_HD int ra_plan_ring_block32(int P, int rank, int s) {
  int j = (rank - s) % P;
  return j < 0 ? j + P : j;
}

// Workgroups are handed to the 8 XCDs round-robin (hardware workgroup bid
// runs on XCD bid % 8, the (bid / 8)-th there).  Logical workgroup of bid,
// for a grid of nwg whose logical order runs through one head's tiles (which
// stream the same K/V or Q/dO tiles) in runs of `run`: XCD x gets
// per = nwg / 8 logical workgroups, so that a head's tiles stay on as few
// XCDs as possible and share their L2.  When a run spans k > 1 XCDs (k the
// least power of two with k * per >= run), the k XCDs of a group take its
// logical range [g k per, (g+1) k per) interleaved (member m gets i k + m),
// so that heavy and light tiles (causal masking) are shared evenly instead of
// one XCD getting all the late tiles.  A bijection on [0, nwg).
RA_HD int ra_plan_xcd_remap(int bid, int nwg, int run) {
  if (nwg % 8 != 0) return bid;
  const int per = nwg / 8, x = bid % 8, i = bid / 8;
  int k = 1;
  while (k < 8 && k * per < run) k *= 2;
  return (x / k) * k * per + i * k + (x % k);
}

// Head (batch * Hq + h) and query tile of logical workgroup l in a grid of
// nwg = nqt * heads, after ra_plan_xcd_remap.  When every XCD holds an even
// number of whole heads, the query tiles of each pair of heads are
// interleaved (h0 t, h1 t, h0 t', h1 t', ...); otherwise a head's tiles are
// consecutive.  Under causal masking later query tiles come first within a
// head.  With one workgroup per CU the dispatcher hands the next workgroup of
// an XCD to the first CU that frees up; interleaving two heads makes the
// light tiles of one batch finish first and pick up the heavy tiles of the
// next (longest-first pairing), so every CU gets the same work.  A bijection
// on [0, nwg) -> (head, tile).
RA_HD void ra_plan_head_tile(int l, int nwg, int nqt, int causal, int* head, int* qt) {
  int hd, qi;
  if (nwg % 8 == 0 && (nwg / 8) % (2 * nqt) == 0) {
    const int pr = l / (2 * nqt), j = l % (2 * nqt);
    hd = 2 * pr + (j & 1);
    qi = j >> 1;
  } else {
    hd = l / nqt;
    qi = l % nqt;
  }
  *head = hd;
  *qt = causal ? nqt - 1 - qi : qi;
}

RA_HD int ra_plan_class(int64_t q0, int64_t nq, int64_t k0, int64_t nk, int causal) {
  if (nq <= 0 || nk <= 0) return RA_CLASS_SKIP;
  if (!causal) return RA_CLASS_FULL;
  const int64_t q_last = q0 + nq - 1, k_last = k0 + nk - 1;
  if (k0 > q_last) return RA_CLASS_SKIP;   // earliest key is after the latest query
  if (k_last <= q0) return RA_CLASS_FULL;  // latest key is at or before the earliest query
  return RA_CLASS_PARTIAL;
}

// Number of key tiles (bn wide) of a block [k0, k0+nk) that hold at least one
// key visible to queries [q0, q0+nq): 0 for SKIP; under causal masking the
// tiles past the last query's position are dropped.
RA_HD int64_t ra_plan_key_tiles(int64_t q0, int64_t nq, int64_t k0, int64_t nk, int causal,
                                int64_t bn) {
  if (ra_plan_class(q0, nq, k0, nk, causal) == RA_CLASS_SKIP) return 0;
  int64_t n = nk;
  if (causal) {
    const int64_t last_visible = q0 + nq - 1 - k0;  // >= 0 here
    if (last_visible + 1 < n) n = last_visible + 1;
  }
  return (n + bn - 1) / bn;
}

// Mask decision of a run of bn key slots holding nvalid keys (nvalid <= bn),
// the first at relative position rel = (its global position) - q0, for the
// queries at global positions q0, q0 + 1, ...: the run needs the masked
// softmax unless all bn keys exist and, under causal masking, the last lies
// at or before q0 (then every key is visible to every query from q0 on, the
// pair is FULL).  I is the integer type of the caller (the kernels pass
// 32-bit relative positions saturated at +-2^30, which keeps the sign).
template <typename I>
RA_HD bool ra_plan_tile_masked(I rel, I nvalid, I bn, int causal) {
  return nvalid < bn || (causal && rel + bn - 1 > 0);
}

// Keys visible to the query at global position q in a run of nvalid keys
// from global position k0: always a prefix, keys k0 .. k0 + lim - 1.
RA_HD int64_t ra_plan_visible_prefix(int64_t q, int64_t k0, int64_t nvalid, int causal) {
  if (!causal) return nvalid;
  const int64_t vis = q - k0 + 1;
  return vis < nvalid ? (vis > 0 ? vis : 0) : nvalid;
}

// Valid keys of slot half hf (0 or 1) of a run of nvalid keys of 2 * half
// slots (a 64-key tile processed as two 32-key units).
RA_HD int ra_plan_half_valid(int nvalid, int hf, int half) {
  const int x = nvalid - half * hf;
  return x < 0 ? 0 : (x > half ? half : x);
}

// First of nu units of 32 queries (unit v from global position q0 + 32 v)
// that the 32 keys klast - 31 .. klast (one wave of the dK/dV kernel) see
// in full, or nu when none does: every key lies before the key end kv_end
// and, under causal masking, at or before the unit's first query.  The
// units before it take the per-element test.
RA_HD int ra_plan_first_full_unit(int64_t klast, int64_t kv_end, int64_t q0, int nu, int causal) {
  if (klast >= kv_end) return nu;
  if (!causal) return 0;
  const int64_t d = klast - q0;  // unit v is seen in full iff d <= 32 v
  if (d <= 0) return 0;
  const int64_t v = (d + 31) / 32;
  return v < nu ? (int)v : nu;
}

// First query tile (bn rows, from local row 0 at global position qpos, nqc
// rows) that sees the key at global position kfirst, or the tile count when
// none does: under causal masking the rows before kfirst see no key at or
// after it; without masking every row sees every key.
RA_HD int ra_plan_first_query_tile(int64_t kfirst, int64_t qpos, int nqc, int bn, int causal) {
  const int ntq = (nqc + bn - 1) / bn;
  int64_t qlo = causal ? kfirst - qpos : 0;
  qlo = qlo < 0 ? 0 : qlo;
  return qlo >= nqc ? ntq : (int)(qlo / bn);
}

