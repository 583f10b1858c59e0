// ra_kernels.hip -- gfx950 kernels of libringattn.
//
// What is computed (glossary page "sequence parallelism transformers"):
// section "Ring Attention", item "Computation" -- a rank attends its local
// queries to each key/value block it holds and accumulates; section
// "Implementation Considerations", item "Numerical Stability" -- the softmax
// normalisation is carried across blocks as a running max m and running sum l
// per query row; section "Flash Attention with Sequence Parallelism", item
// "Tiled Computation" -- each block is processed in tiles that stay on chip.
//
// bf16 path (attn_bf16_kernel): one workgroup = 8 waves = 256 query rows of
// one head; each wave owns 32 query rows.  Per key tile of 64 keys:
//   S^T (keys x queries) = K Q^T   v_mfma_f32_32x32x16_bf16; K from LDS is the
//                                  A operand, the Q fragment stays in VGPRs
//                                  for the whole kernel as the B operand
//   online softmax                 the accumulator layout puts one query per
//                                  lane (lane & 31) and 32 of its 64 keys in
//                                  that lane's registers; the other 32 sit in
//                                  lane ^ 32, so the row max needs one
//                                  v_permlane32_swap and the rescale factor is
//                                  a per-lane scalar
//   O^T (channels x queries) += V^T P^T   P^T goes from the S^T accumulator
//                                  registers straight into the B operand
//                                  (bf16, round to nearest even); the A
//                                  operand V^T comes from row-major V in LDS
//                                  through the transposing ds_read_b64_tr_b16
// K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no register
// staging) into two stages, row-major under an XOR swizzle of the 16-byte
// slots (conflict-free K and transposing V reads); one barrier per tile.
// Logits are scaled in fp32 (never folded into bf16 Q); exponentials are
// base 2 with the scale folded into one FMA: p = exp2(s * scale * log2(e) - m2),
// m2 the running max in log2 units.  m2 is moved only when a tile's max
// exceeds it by more than kLazyTau, so the rescale of O is rare; the result
// does not depend on which max is used as long as o, l and m agree
// (O = o / l, LSE = m + ln l), and p stays <= 2^kLazyTau.
//
// fp32 path (attn_f32_kernel): one wave per 64 query rows, fp32 FMA
// throughout, for the fp32 workloads.
#include "ra_launch.h"
#include "ra_plan.h"

#include <type_traits>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are handed to the 8 XCDs round-robin.  Give XCD x the contiguous
// logical range [x * n/8, (x+1) * n/8) so that all query tiles of a head (and
// the heads sharing a kv head) run on one XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  if (nwg % 8 != 0) return bid;
  return (bid % 8) * (nwg / 8) + bid / 8;
}

// ---------------------------------------------------------------------------
// bf16 path.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr float kLazyTau = 8.0f;

// Physical 16-byte slot of logical slot p in LDS row r: p ^ f(r), with
// f(r) = 4 (r & 3) + ((r >> 2) & 3) (the two low 2-bit fields of r swapped),
// cut to the row's slot count.  With 64 LDS banks (256 bytes per cycle) a
// 128-bit read of 16 consecutive rows at one logical slot, and a transposing
// 64-bit read of 4 consecutive rows (aligned to 4) at 4 consecutive slots
// (aligned to 4), both touch 16 different 16-byte bank groups.  f depends on
// r & 15 only, so row offsets that are multiples of 16 keep the pattern.
template <int SLOTS>
__device__ __forceinline__ int swz(int r, int p) {
  return p ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (SLOTS - 1));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [I, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int D>
__global__ void __launch_bounds__(512, 1) attn_bf16_kernel(RaAttnArgs a) {
  constexpr int NW = 8, BM = NW * 32, BN = RA_BF16_BN, NT = NW * 64;
  constexpr int SLOTS = D / 8;                 // 16-byte slots per row
  constexpr int TILE_BYTES = BN * D * 2;       // one K or V tile
  constexpr int NI = BN * SLOTS / NT;          // direct-load instructions per thread per tile
  static_assert(NI * NT == BN * SLOTS, "tile split");
  static_assert(BN == 64, "the softmax below is written for two 32-key halves");
  // [0], [1]: K stages; [2], [3], [4]: V stages
  __shared__ __attribute__((aligned(1024))) char smem[5][TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: keep it (and the schedule built on it) in SGPRs
  const int wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;

  const int nqt = (a.nq + BM - 1) / BM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int qt = logical % nqt;
  const int hb = logical / nqt;
  const int h = hb % a.Hq, b = hb / a.Hq;
  if (a.causal) qt = nqt - 1 - qt;  // later query tiles see more keys: start them first
  const int hk = h / (a.Hq / a.Hkv);

  const int qrow_wg = qt * BM;
  const int qrow_w = qrow_wg + wave * 32;
  const int my_q = qrow_w + lr;
  const bool q_ok = my_q < a.nq;

  // Q fragment (B operand of S^T = K Q^T): lane holds Q[my_q][16c + 8lg .. +7].
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)my_q * a.q_ss +
                       (int64_t)h * a.q_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_ok) w = *(const u32x4*)(qp + 16 * c);
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Running state.  o[db][r] = O^T[32db + 8(r/4) + 4lg + r%4][my_q] (unnormalised);
  // m2 = running max of s * c (log2 units); lsum = this lane's half of the row sum.
  f32x16 o[D / 32];
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  if (a.state_in && q_ok) {
    const float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x = *(const f32x4*)(op + 32 * db + 8 * j + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][4 * j + i] = x[i];
      }
    const float mv = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss];
    const float lv = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss];
    m2 = mv * kLog2e;  // -inf stays -inf
    lsum = lg == 0 ? lv : 0.f;
  }

  const int64_t q0_wg = a.q_off + qrow_wg;
  const int nq_wg = min(BM, a.nq - qrow_wg);
  const int nsteps = a.ring ? a.P : 1;
  // Key position (ring mode: also first row in k/v) of the block folded at
  // loop step s.  The blocks arrive in ring order (block (rank - s) mod P at
  // ring step s); the rank's own block (ring step 0) is resident from the
  // start and is folded last.  Every other block is then walked in lockstep
  // by all query tiles of a head (the own block's causal tile count differs
  // per query tile and would spread them apart), which keeps the K/V stream
  // they share in L2.  The merge is order-independent: only rounding changes.
  auto step_kv_off = [&](int s) -> int64_t {
    return a.ring ? (int64_t)ra_plan_ring_block32(a.P, a.rank, (s + 1) % a.P) * a.nkv : a.kv_off;
  };
  auto step_tiles = [&](int s) -> int {
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, step_kv_off(s), a.nkv, a.causal, BN);
  };

  // Direct loads of one key tile.  Each tile is loaded by one group of four
  // waves, 2 NI instructions each: K by waves 4-7, V by waves 0-3, each in its
  // softmax phase.  Lane L of instruction inst = (wave & 3) 2 NI + i fills
  // physical slot inst * 64 + L of the tile (row r, physical slot p) and loads
  // the logical slot that the swizzle puts there.  The global address is a
  // uniform tile base plus a per-lane 32-bit offset fixed for the kernel.  In
  // the last tile of a block, rows past the block end re-read the last valid
  // row (finite data; masked in S, zero weight in P).
  const char* gbase = (wave >> 2) ? (const char*)a.k + 2 * ((int64_t)b * a.k_sb + (int64_t)hk * a.k_sh)
                                  : (const char*)a.v + 2 * ((int64_t)b * a.v_sb + (int64_t)hk * a.v_sh);
  const int64_t gstride = (wave >> 2) ? a.k_ss : a.v_ss;  // elements; 64 rows fit 32-bit offsets
  auto gslot = [&](int i, int& r) -> unsigned {
    const int ls = ((wave & 3) * 2 * NI + i) * 64 + lane;
    r = ls / SLOTS;
    return 16u * (unsigned)swz<SLOTS>(r, ls % SLOTS);
  };
  unsigned goff[2 * NI];
#pragma unroll
  for (int i = 0; i < 2 * NI; ++i) {
    int r;
    const unsigned sl = gslot(i, r);
    goff[i] = (unsigned)r * (unsigned)gstride * 2u + sl;
  }
  // row0: first row of the tile in k/v; nvalid: rows of the tile inside the block
  auto issue = [&](int64_t row0, int nvalid, int stage) {
    const char* tb = gbase + row0 * gstride * 2;
    if (nvalid == BN) {
#pragma unroll
      for (int i = 0; i < 2 * NI; ++i)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(tb + goff[i]),
                                         (lds_void_t*)(&smem[stage][((wave & 3) * 2 * NI + i) * 1024]), 16, 0, 0);
    } else {
      const int last = nvalid - 1;
#pragma unroll
      for (int i = 0; i < 2 * NI; ++i) {
        int r;
        const unsigned sl = gslot(i, r);
        const unsigned off = (unsigned)(r < last ? r : last) * (unsigned)gstride * 2u + sl;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(tb + off),
                                         (lds_void_t*)(&smem[stage][((wave & 3) * 2 * NI + i) * 1024]), 16, 0, 0);
      }
    }
  };

  // Per-lane LDS byte offsets inside a K or V tile (rows of 2D bytes).
  // K, A operand of S^T for key block bb: row 32 bb + lr, logical slot 2c + lg:
  //   koff[c] + 64 D bb.
  int koff[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) koff[c] = lr * 2 * D + 16 * swz<SLOTS>(lr, 2 * c + lg);
  // V, transposing reads for key block bb, half hh, second 8 rows (+8): source
  // lane j = lane % 16 supplies row 32 bb + 16 hh + 8 half + 4 (lane / 32) + j / 4
  // and the 8 bytes at channel 32 db + 16 ((lane / 16) % 2) + 4 (j % 4), i.e.
  // logical slot 4 db + 2 ((lane / 16) % 2) + (j % 4) / 2, byte 8 (j % 2):
  //   voff[half][db] + 2D (32 bb + 16 hh).
  const int vj = lane & 15, ve = vj >> 2, vc = vj & 3, vgrp = lane >> 4;
  const int vx = 2 * (vgrp & 1) + (vc >> 1);
  const unsigned smem_lds = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)&smem[0][0]);
  unsigned voff[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int r = 4 * lg + ve + 8 * half;
      voff[half][db] = smem_lds + 2 * TILE_BYTES + r * 2 * D + 16 * swz<SLOTS>(r, 4 * db + vx) + 8 * (vc & 1);
    }

  // ---- schedule ----------------------------------------------------------
  // The workgroup's key tiles c_0 .. c_{n-1} (ring order, causal tiles past
  // the last query dropped) are processed in two phases each:
  //   MFMA phase j:  S(j) = K(c_j) Q^T;  O^T += V(c_{j-1})^T P(j-1)^T
  //   VALU phase j:  mask, row max, lazy rescale, P(j) = exp2(S(j) c - m), l
  // Waves 0-3 run phase index (phi) as their own; waves 4-7 run one phase
  // behind, so on every SIMD (waves w and w + 4) one wave issues MFMAs while
  // the other does the softmax.  Every phase ends with a barrier.  K(c_k) is
  // read in phases 2k and 2k+1, V(c_{k-1}) in the same two phases; the
  // direct loads of K(c_{k+1}) and V(c_k) are issued at the start of phase
  // 2k into the stages freed by phase 2k-1 and waited for before the barrier
  // that ends phase 2k+1.  All waves run the same 2n + 2 barriers.
  int n = 0;
  for (int s = 0; s < nsteps; ++s) n += step_tiles(s);

  if (n > 0) {  // workgroup-uniform
    const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7
    // Load cursor: step ls, tile lu, with the step's tile count, key position
    // and first row cached.  It walks c_0, c_1, ... once; the V load of c_k
    // reuses the row and valid count of its K load, and the softmax of c_j
    // reads the key position and valid count recorded with K(c_j).
    int ls = 0;
    while (step_tiles(ls) == 0) ++ls;
    int lu = 0, lnt = step_tiles(ls);
    int64_t lkv = step_kv_off(ls);
    int64_t lrow = a.ring ? lkv : 0;
    auto cur_nvalid = [&]() -> int {
      const int64_t left = a.nkv - (int64_t)lu * BN;
      return left < BN ? (int)left : BN;
    };
    auto cur_row = [&]() -> int64_t { return lrow + (int64_t)lu * BN; };
    auto cur_pos = [&]() -> int64_t { return lkv + (int64_t)lu * BN; };
    auto step_cursor = [&]() {
      if (++lu < lnt) return;
      lu = 0;
      do {
        ++ls;
      } while (ls < nsteps && (lnt = step_tiles(ls)) == 0);
      if (ls < nsteps) {
        lkv = step_kv_off(ls);
        lrow = a.ring ? lkv : 0;
      }
    };
    // row / valid count of the tile whose V is issued next; (position, valid
    // count) of tiles c_j with j even (hpos0, hval0) and odd (hpos1, hval1)
    int64_t vrow = cur_row(), hpos0 = cur_pos(), hpos1 = 0, npos = 0;
    int vval = cur_nvalid(), hval0 = vval, hval1 = 0;
    issue(vrow, vval, grp ? 0 : 2);  // K(c_0) by waves 4-7, V(c_0) by waves 0-3
    step_cursor();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    f32x16 sacc[2];
    bf16x8 pf[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sacc[bb] = f32x16{};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pf[bb][hh] = bf16x8{};
    }

    for (int phi = 0; phi <= 2 * n + 1; ++phi) {
      // Loads.  Phase 2k: waves 4-7 issue K(c_{k+1}) (into the K stage read in
      // phases 2k-2, 2k-1).  Phase 2k+1: waves 0-3 issue V(c_{k+1}) (into V
      // stage (k+1) % 3, read in phases 2k-2, 2k-1).  (vrow, vval) describe
      // c_{k+1} from phase 2k on.
      bool v_issued = false;
      if (!(phi & 1) && (phi >> 1) + 1 < n) {
        const int k = phi >> 1;
        vrow = cur_row();
        vval = cur_nvalid();
        npos = cur_pos();
        if (grp == 1) issue(vrow, vval, (k + 1) & 1);
        step_cursor();
      }
      if ((phi & 1) && (phi >> 1) + 1 < n && grp == 0) {
        issue(vrow, vval, 2 + ((phi >> 1) + 1) % 3);
        v_issued = true;
      }
      const int my = phi - grp;
      if (my >= 0) {
        const int j = my >> 1;
        if (!(my & 1)) {
          // ---- MFMA phase j ----
          if (j < n) {
            // all K fragments of the tile first, then the MFMAs, so the LDS
            // latency is paid once per tile rather than once per MFMA
            const char* Ks = smem[j & 1];
            bf16x8 kf[2][D / 16];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
              for (int c = 0; c < D / 16; ++c) kf[bb][c] = *(const bf16x8*)(Ks + koff[c] + 64 * D * bb);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
              sacc[bb] = f32x16{};
#pragma unroll
              for (int c = 0; c < D / 16; ++c)
                sacc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[bb][c], qf[c], sacc[bb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);  // the LDS reads first
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 16), 0);  // then the MFMAs
          }
          if (j >= 1) {
            // O^T += V^T P^T of tile j-1.  The transposing reads are inline
            // asm so the compiler does not order them behind the in-flight
            // direct loads (it cannot prove they do not alias); the wait that
            // follows carries their registers, so the MFMAs stay behind it.
            const unsigned vst = (unsigned)((j - 1) % 3) * TILE_BYTES;
            u32x2 lo[2][D / 32], hi[2][D / 32];
#define RA_TR_READ(BUF, G, DB)                                                                   \
  if constexpr (DB < D / 32) {                                                                   \
    constexpr int off = (32 * ((G) >> 1) + 16 * ((G) & 1)) * 2 * D;                             \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo[BUF][DB]) : "v"(voff[0][DB] + vst), "i"(off)); \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi[BUF][DB]) : "v"(voff[1][DB] + vst), "i"(off)); \
  }
#define RA_TR_GROUP(BUF, G) RA_TR_READ(BUF, G, 0) RA_TR_READ(BUF, G, 1) RA_TR_READ(BUF, G, 2) RA_TR_READ(BUF, G, 3)
#define RA_TR_WAIT(BUF, N)                                                                       \
  if constexpr (D == 128)                                                                        \
    asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(lo[BUF][0]), "+v"(hi[BUF][0]), "+v"(lo[BUF][1]), \
                 "+v"(hi[BUF][1]), "+v"(lo[BUF][2]), "+v"(hi[BUF][2]), "+v"(lo[BUF][3]), "+v"(hi[BUF][3])); \
  else                                                                                           \
    asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(lo[BUF][0]), "+v"(hi[BUF][0]), "+v"(lo[BUF][1]), \
                 "+v"(hi[BUF][1]));
#define RA_PV(BUF, G)                                                                            \
  _Pragma("unroll") for (int db = 0; db < D / 32; ++db) {                                        \
    const u32x4 w = {lo[BUF][db][0], lo[BUF][db][1], hi[BUF][db][0], hi[BUF][db][1]};            \
    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),               \
                                                    pf[(G) >> 1][(G) & 1], o[db], 0, 0, 0);      \
  }
            // O^T += V^T P^T of tile j-1, four (key block, half) groups; the
            // reads of group g+1 are in flight while group g's MFMAs issue.
            // The transposing reads are inline asm so the compiler does not
            // order them behind the in-flight direct loads (it cannot prove
            // they do not alias); each wait carries the registers it
            // guarantees, so the MFMAs stay behind it.  lgkmcnt counts only
            // these reads here (LDS completes in order; scalar loads only add).
            if constexpr (D == 128) {
              RA_TR_GROUP(0, 0)
              RA_TR_GROUP(1, 1)
              RA_TR_WAIT(0, 8)
              RA_PV(0, 0)
              RA_TR_GROUP(0, 2)
              RA_TR_WAIT(1, 8)
              RA_PV(1, 1)
              RA_TR_GROUP(1, 3)
              RA_TR_WAIT(0, 8)
              RA_PV(0, 2)
              RA_TR_WAIT(1, 0)
              RA_PV(1, 3)
            } else {
              RA_TR_GROUP(0, 0)
              RA_TR_GROUP(1, 1)
              RA_TR_WAIT(0, 4)
              RA_PV(0, 0)
              RA_TR_GROUP(0, 2)
              RA_TR_WAIT(1, 4)
              RA_PV(1, 1)
              RA_TR_GROUP(1, 3)
              RA_TR_WAIT(0, 4)
              RA_PV(0, 2)
              RA_TR_WAIT(1, 0)
              RA_PV(1, 3)
            }
#undef RA_PV
#undef RA_TR_WAIT
#undef RA_TR_GROUP
#undef RA_TR_READ
          }
        } else if (j < n) {
          // ---- VALU phase j: softmax of tile c_j ----
          const int64_t k0 = (j & 1) ? hpos1 : hpos0;
          const int nvalid = (j & 1) ? hval1 : hval0;
          const int64_t q0w = a.q_off + qrow_w;
          const int nqw = min(32, a.nq - qrow_w);
          const int cls = ra_plan_class(q0w, nqw, k0, nvalid, a.causal);
          if (cls != RA_CLASS_FULL || nvalid < BN) {
            // Keys kvi < lim of this tile are visible to this lane's query:
            // lim = valid keys, cut at the query's own position under causal
            // masking, 0 for SKIP (no visible key for these rows: p = 0).  The
            // key index of register r is 32 bb + 8 (r / 4) + (r % 4) + 4 lg.
            int64_t lim64 = cls == RA_CLASS_SKIP ? 0 : nvalid;
            if (a.causal) {
              const int64_t vis = q0w + lr - k0 + 1;
              lim64 = vis < lim64 ? (vis > 0 ? vis : 0) : lim64;
            }
            const int lim = (int)lim64 - 4 * lg;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                sacc[bb][r] = (32 * bb + 8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : sacc[bb][r];
          }
          float mx = -INFINITY;
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[bb][r]);
          {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          }
          const float t = mx * a.c;
          const bool bump = t > m2 + kLazyTau;  // move the max only when it grows by more than kLazyTau
          if (__builtin_amdgcn_ballot_w64(bump)) {
            const float alpha = bump ? fast_exp2(m2 - t) : 1.f;  // 0 when m2 was -inf
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m2 = bump ? t : m2;
          }
          const float m_use = m2 == -INFINITY ? 0.f : m2;  // no visible key yet: p = 0
          // The row sum takes the fp32 p (only the MFMA operand is rounded to
          // bf16): rows with few visible keys would otherwise carry the 2^-9
          // rounding of one term into l and the LSE.
          float psum = 0.f;
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int t8 = 0; t8 < 8; ++t8) {
                const float p = fast_exp2(fmaf(sacc[bb][8 * hh + t8], a.c, -m_use));
                psum += p;
                pf[bb][hh][t8] = (__bf16)p;
              }
          lsum += psum;
        }
      }
      // c_{k+1}'s position and valid count go into its history slot only now:
      // waves 4-7 read c_{k-1}'s (same slot) earlier in this phase.
      if (!(phi & 1) && (phi >> 1) + 1 < n) {
        if (((phi >> 1) + 1) & 1) {
          hpos1 = npos;
          hval1 = vval;
        } else {
          hpos0 = npos;
          hval0 = vval;
        }
      }
      // Phase barrier.  Only the odd ones publish LDS data (the direct loads
      // issued two phases earlier), so only they wait for vmcnt; the even
      // ones just order this phase's LDS reads before the next loads.  Inline
      // asm with a memory clobber keeps the compiler from moving LDS accesses
      // across it (and from adding its own full waits).
      // Odd barriers publish the loads issued two phases earlier: K(c_{k+1})
      // of waves 4-7 (phase 2k) and V(c_k) of waves 0-3 (phase 2k-1); a V
      // group issued in this phase may stay in flight.
      if (phi < 2 * n + 1) {
        if (!(phi & 1))
          asm volatile("s_barrier" ::: "memory");
        else if (v_issued)
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NI) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
  }

  // Epilogue: the two halves of each row sum live in lanes lr and lr + 32.
  float ltot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!q_ok) return;
  if (a.out_state) {
    float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x = {o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
        *(f32x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
      }
    if (lg == 0) {
      a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss] = m2 * kLn2;
      a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss] = ltot;
    }
  } else {
    const float inv = 1.f / ltot;
    const int64_t base = (int64_t)b * a.o_sb + (int64_t)my_q * a.o_ss + (int64_t)h * a.o_sh;
    if (a.o_bf16) {
      __bf16* op = (__bf16*)a.o + base;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 x = {(__bf16)(o[db][4 * j] * inv), (__bf16)(o[db][4 * j + 1] * inv),
                      (__bf16)(o[db][4 * j + 2] * inv), (__bf16)(o[db][4 * j + 3] * inv)};
          *(bf16x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
        }
    } else {
      float* op = (float*)a.o + base;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 x = {o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                     o[db][4 * j + 3] * inv};
          *(f32x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
        }
    }
    if (lg == 0 && a.lse)
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)my_q * a.lse_ss] =
          (m2 + __log2f(ltot)) * kLn2;
  }
}

// fp32 path: one wave per workgroup, one query row per lane, fp32 FMA
// throughout (dot products, softmax, P V).  K and V tiles of 64 keys are
// staged in LDS and read by all lanes at the same address (broadcast).
template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(RaAttnArgs a) {
  constexpr int BM = RA_F32_BM, BN = RA_F32_BN;
  __shared__ __attribute__((aligned(16))) float Ks[BN * D];
  __shared__ __attribute__((aligned(16))) float Vs[BN * D];
  const int tid = threadIdx.x;
  const int nqt = (a.nq + BM - 1) / BM;
  int qt = blockIdx.x % nqt;
  const int hb = blockIdx.x / nqt;
  const int h = hb % a.Hq, b = hb / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int my_q = qt * BM + tid;
  const bool q_ok = my_q < a.nq;

  float q[D], o[D];
  {
    const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)my_q * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (q_ok) x = *(const f32x4*)(qp + c);
      q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
    }
  }
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  if (a.state_in && q_ok) {
    const float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4 x = *(const f32x4*)(op + c);
      o[c] = x[0]; o[c + 1] = x[1]; o[c + 2] = x[2]; o[c + 3] = x[3];
    }
    m2 = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss] * kLog2e;
    lsum = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss];
  }

  const int64_t q0_wg = a.q_off + (int64_t)qt * BM;
  const int nq_wg = min(BM, a.nq - qt * BM);
  const int nsteps = a.ring ? a.P : 1;
  for (int s = 0; s < nsteps; ++s) {
    const int64_t jb = a.ring ? ra_plan_ring_block(a.P, a.rank, s) : 0;
    const int64_t kv_off = a.ring ? jb * a.nkv : a.kv_off;
    const int64_t row0 = a.ring ? jb * a.nkv : 0;
    const int nt = (int)ra_plan_key_tiles(q0_wg, nq_wg, kv_off, a.nkv, a.causal, BN);
    for (int u = 0; u < nt; ++u) {
      const int64_t left = a.nkv - (int64_t)u * BN;
      const int nvalid = left < BN ? (int)left : BN;
      const float* kb = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh + (row0 + (int64_t)u * BN) * a.k_ss;
      const float* vb = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh + (row0 + (int64_t)u * BN) * a.v_ss;
      __syncthreads();
      for (int id = tid; id < BN * D / 4; id += 64) {
        const int row = id / (D / 4), c4 = id % (D / 4);
        f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
        if (row < nvalid) {
          kx = *(const f32x4*)(kb + (int64_t)row * a.k_ss + 4 * c4);
          vx = *(const f32x4*)(vb + (int64_t)row * a.v_ss + 4 * c4);
        }
        *(f32x4*)(Ks + row * D + 4 * c4) = kx;
        *(f32x4*)(Vs + row * D + 4 * c4) = vx;
      }
      __syncthreads();
      const int64_t k0 = kv_off + (int64_t)u * BN;
      const int64_t qpos = a.q_off + my_q;
      float sc[BN];
      float mx = -INFINITY;
      for (int j = 0; j < BN; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) dot = fmaf(q[c], Ks[j * D + c], dot);
        const bool vis = j < nvalid && (!a.causal || k0 + j <= qpos);
        sc[j] = vis ? dot : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float m_new = fmaxf(m2, mx * a.c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m2 - m_use);
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
      for (int j = 0; j < BN; ++j) {
        const float p = exp2f(fmaf(sc[j], a.c, -m_use));
        lsum += p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = fmaf(p, Vs[j * D + c], o[c]);
      }
      m2 = m_new;
    }
  }

  if (!q_ok) return;
  if (a.out_state) {
    float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
    for (int c = 0; c < D; c += 4) *(f32x4*)(op + c) = f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]};
    a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss] = m2 * kLn2;
    a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss] = lsum;
  } else {
    const float inv = 1.f / lsum;
    const int64_t base = (int64_t)b * a.o_sb + (int64_t)my_q * a.o_ss + (int64_t)h * a.o_sh;
    if (a.o_bf16) {
      __bf16* op = (__bf16*)a.o + base;
#pragma unroll
      for (int c = 0; c < D; c += 4)
        *(bf16x4*)(op + c) = bf16x4{(__bf16)(o[c] * inv), (__bf16)(o[c + 1] * inv),
                                    (__bf16)(o[c + 2] * inv), (__bf16)(o[c + 3] * inv)};
    } else {
      float* op = (float*)a.o + base;
#pragma unroll
      for (int c = 0; c < D; c += 4)
        *(f32x4*)(op + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
    }
    if (a.lse)
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)my_q * a.lse_ss] =
          m2 * kLn2 + logf(lsum);
  }
}

// O = o_acc / l and LSE = m + ln l; one thread per 4 channels of a row, rows
// in [B, S, H] order so consecutive threads touch consecutive 16-byte chunks.
__global__ void __launch_bounds__(256) finalize_kernel(RaFinArgs a) {
  const int nd4 = a.d / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.S * a.H * nd4;
  if (idx >= total) return;
  const int c4 = (int)(idx % nd4);
  const int64_t row = idx / nd4;
  const int h = (int)(row % a.H);
  const int64_t t = row / a.H;
  const int s = (int)(t % a.S), b = (int)(t / a.S);
  const float lv = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)s * a.l_ss];
  const f32x4 x = *(const f32x4*)(a.oacc + (int64_t)b * a.oa_sb + (int64_t)s * a.oa_ss + (int64_t)h * a.oa_sh + 4 * c4);
  const float inv = 1.f / lv;
  const int64_t ob = (int64_t)b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)h * a.o_sh + 4 * c4;
  if (a.o_bf16)
    *(bf16x4*)((__bf16*)a.o + ob) = bf16x4{(__bf16)(x[0] * inv), (__bf16)(x[1] * inv),
                                          (__bf16)(x[2] * inv), (__bf16)(x[3] * inv)};
  else
    *(f32x4*)((float*)a.o + ob) = f32x4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
  if (c4 == 0 && a.lse) {
    const float mv = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)s * a.m_ss];
    a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)s * a.lse_ss] = mv + logf(lv);
  }
}

__global__ void __launch_bounds__(256) init_kernel(RaInitArgs a) {
  const int nd4 = a.d / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.S * a.H * nd4;
  if (idx >= total) return;
  const int c4 = (int)(idx % nd4);
  const int64_t row = idx / nd4;
  const int h = (int)(row % a.H);
  const int64_t t = row / a.H;
  const int s = (int)(t % a.S), b = (int)(t / a.S);
  *(f32x4*)(a.oacc + (int64_t)b * a.oa_sb + (int64_t)s * a.oa_ss + (int64_t)h * a.oa_sh + 4 * c4) =
      f32x4{0.f, 0.f, 0.f, 0.f};
  if (c4 == 0) {
    a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)s * a.m_ss] = -INFINITY;
    a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)s * a.l_ss] = 0.f;
  }
}

}  // namespace

hipError_t ra_launch_attn_bf16(const RaAttnArgs& a, int d, hipStream_t st) {
  const int nqt = (a.nq + RA_BF16_BM - 1) / RA_BF16_BM;
  const dim3 grid((unsigned)((int64_t)nqt * a.Hq * a.B)), block(512);
  if (d == 128) hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_attn_f32(const RaAttnArgs& a, int d, hipStream_t st) {
  const int nqt = (a.nq + RA_F32_BM - 1) / RA_F32_BM;
  const dim3 grid((unsigned)((int64_t)nqt * a.Hq * a.B)), block(64);
  if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_finalize(const RaFinArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.B * a.S * a.H * (a.d / 4);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(finalize_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_init(const RaInitArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.B * a.S * a.H * (a.d / 4);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(init_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}
