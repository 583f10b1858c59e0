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
// bf16 path.  Two forms of the same pipeline; the library launches the
// second (attn_bf16_w64_kernel, 64 query rows per wave, one wave per SIMD,
// described where it is defined), which reads half as much from LDS per
// MFMA.  The first (attn_bf16_kernel) is described here: one workgroup = 8
// waves = 256 query rows of one head; each wave owns 32 query rows; the two
// waves that share a SIMD (w and w + 4) feed its matrix core and vector ALU
// from two instruction streams.  Keys come in tiles of 64, processed as two
// 32-key units:
//   S^T (keys x queries) = K Q^T   v_mfma_f32_32x32x16_bf16; K from LDS is the
//                                  A operand, the Q fragment stays in VGPRs
//                                  for the whole kernel as the B operand
//   online softmax                 the accumulator layout puts one query per
//                                  lane (lane & 31) and 16 of the unit's 32
//                                  keys in that lane's registers (the other
//                                  16 sit in lane ^ 32)
//   O^T (channels x queries) += V^T P^T   P^T goes from registers straight
//                                  into the B operand (bf16, round to nearest
//                                  even); the A operand V^T comes from
//                                  row-major V in LDS through the transposing
//                                  ds_read_b64_tr_b16
// Per wave, a software pipeline with one step per unit u: the MFMAs of
// S(u+1) and of O += V(u-1) P(u-1) interleaved with the vector work of the
// softmax of S(u), which depends on neither.
// K and V tiles move HBM -> LDS with buffer loads straight into LDS (no
// register staging), loaded three (K) and two (V) tiles ahead into four K
// and four V stages, row-major under an XOR swizzle of the 16-byte slots
// (conflict-free K and transposing V reads); one barrier per tile.  The
// loop body covers four tiles, so every LDS read address is a per-lane base
// plus an immediate offset.
// Logits are scaled in fp32 (never folded into bf16 Q); exponentials are
// base 2 with the scale folded into one FMA: p = exp2(s * scale * log2(e) - m2),
// m2 the running max in log2 units.  The softmax uses m2 as it stands and
// skips the row max; a unit whose row sum exceeds kRedoSum = 2^8, or is not
// finite, is redone against its exact row max, which becomes m2 (with O and
// l rescaled).  The result does not depend on which max is used as long as
// o, l and m agree (O = o / l, LSE = m + ln l), and p stays at most 2^8.
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
// max of three without the NaN canonicalisation fmaxf brings along (the
// inputs are MFMA results or -inf, never signalling NaNs)
__device__ __forceinline__ float vmax3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

// ---------------------------------------------------------------------------
// bf16 path.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr float kRedoSum = 256.0f;  // redo a unit when a lane's sum of p exceeds this

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

// Position in the workgroup's key tile sequence: loop step s, tile u of the
// step's nt tiles, the step's first key position kv.
struct TileCursor {
  int s, u, nt;
  int64_t kv;
};

template <int D>
__global__ void __launch_bounds__(512, 1) attn_bf16_kernel(RaAttnArgs a) {
  constexpr int NW = 8, BM = NW * 32, BN = RA_BF16_BN;
  constexpr int SLOTS = D / 8;                 // 16-byte slots per row
  constexpr int TILE_BYTES = BN * D * 2;       // one K or V tile
  constexpr int NL = TILE_BYTES / 1024 / NW;   // 1 KiB direct loads per wave per tile
  constexpr int KC = D / 16;                   // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                   // 32-channel blocks of O^T
  static_assert(NL * 1024 * NW == TILE_BYTES, "tile split");
  static_assert(BM == RA_BF16_BM && BN == 64, "64-key tiles, processed as two 32-key units");
  // [0] .. [3]: K stages; [4] .. [7]: V stages (tile c_t in K and V stage t % 4)
  __shared__ __attribute__((aligned(1024))) char smem[8][TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep per-wave values in SGPRs
  const int lr = lane & 31, lg = lane >> 5;

  // query tiles: nqt_c per chunk of nqc rows (one chunk unless the share is split)
  const int nqc = a.nsplit == 2 ? (int)a.qc : a.nq;
  const int nqt_c = (nqc + BM - 1) / BM;
  const int nqt = (a.nsplit == 2 ? 2 : 1) * nqt_c;
  int hb, qt;  // later query tiles see more keys under causal masking: they start first
  ra_plan_head_tile(ra_plan_xcd_remap(blockIdx.x, gridDim.x, nqt), gridDim.x, nqt, a.causal, &hb, &qt);
  const int h = hb % a.Hq, b = hb / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int chunk = qt / nqt_c;
  const int64_t qpos0 = chunk ? a.q_off2 : a.q_off;  // global position of the chunk's first row
  const int rank_e = chunk ? a.rank2 : a.rank;        // its ring order

  const int qrow_wg = (qt - chunk * nqt_c) * BM;      // rows within the chunk
  const int qrow_w = qrow_wg + wave * 32;
  const int my_q = chunk * nqc + qrow_w + lr;         // local row (q, o, lse, state)
  const bool q_ok = qrow_w + lr < nqc;

  // Q fragment (B operand of S^T = K Q^T): lane holds Q[my_q][16c + 8lg .. +7].
  bf16x8 qf[KC];
  {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)(q_ok ? my_q : 0) * a.q_ss +
                       (int64_t)h * a.q_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_ok) w = *(const u32x4*)(qp + 16 * c);
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Running state.  o[db][r] = O^T[32db + 8(r/4) + 4lg + r%4][my_q] (unnormalised);
  // m2 = running max of s * c (log2 units); lsum = this lane's half of the row sum.
  f32x16 o[DB];
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  if (a.state_in && q_ok) {
    const float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
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

  const int64_t q0_wg = qpos0 + qrow_wg;
  const int nq_wg = min(BM, nqc - qrow_wg);
  const int nsteps = a.ring ? a.P : 1;
  // Key position (ring mode: also first row in k/v) of the block folded at
  // loop step s.  The blocks arrive in ring order (block (rank - s) mod P at
  // ring step s); the rank's own block (ring step 0) is resident from the
  // start and is folded last.  Every other block is then walked in lockstep
  // by all query tiles of a head (the own block's causal tile count differs
  // per query tile and would spread them apart), which keeps the K/V stream
  // they share in L2.  The merge is order-independent: only rounding changes.
  auto step_kv_off = [&](int s) -> int64_t {
    return a.ring ? (int64_t)ra_plan_ring_block32(a.P, rank_e, (s + 1) % a.P) * a.nkv : a.kv_off;
  };
  // keys of the block at loop step s before the end of the valid keys
  auto step_keys = [&](int s) -> int64_t {
    const int64_t n = a.kv_end - step_kv_off(s);
    return n < 0 ? 0 : (n < a.nkv ? n : a.nkv);
  };
  auto step_tiles = [&](int s) -> int {
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, step_kv_off(s), step_keys(s), a.causal, BN);
  };

  // Direct loads.  All eight waves load a share (NL KiB) of each K and V
  // tile: lane L of instruction inst = wave NL + i fills physical slot
  // inst * 64 + L of the tile (row r, physical slot p) and loads the logical
  // slot that the swizzle puts there.  The loads are buffer loads: a scalar
  // descriptor based at the tile's first row plus a per-lane 32-bit offset
  // fixed for the kernel.  The descriptor's range ends with the tile's last
  // valid row, so in the last tile of a block the rows past the block end
  // are out of range: the buffer unit fetches nothing for them and writes
  // zeros to their LDS bytes (range checked per dword; measured on gfx950),
  // with no branch in the loop.  Those zero rows are masked in S and have
  // zero weight in P.
  const char* kbase = (const char*)a.k + 2 * ((int64_t)b * a.k_sb + (int64_t)hk * a.k_sh);
  const char* vbase = (const char*)a.v + 2 * ((int64_t)b * a.v_sb + (int64_t)hk * a.v_sh);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto gslot = [&](int i, int& r) -> unsigned {
    const int ls = (wv * NL + i) * 64 + lane;
    r = ls / SLOTS;
    return 16u * (unsigned)swz<SLOTS>(r, ls % SLOTS);
  };
  unsigned koffg[NL], voffg[NL];  // row strides of k and v: at most 2^24 elements
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    int r;
    const unsigned sl = gslot(i, r);
    koffg[i] = (unsigned)r * (unsigned)a.k_ss * 2u + sl;
    voffg[i] = (unsigned)r * (unsigned)a.v_ss * 2u + sl;
  }
  // Tile at address tb (row stride `stride` elements) with nvalid valid rows
  // into LDS stage `stage`.
  const unsigned smem_lds = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)&smem[0][0]);
  auto issue = [&](const char* tb, int64_t stride, const unsigned* goff, int nvalid, auto STAGE)
      __attribute__((always_inline)) {
    // range: through the end of row nvalid - 1 (nvalid >= 1; at most
    // 63 * 2^25 + 2D bytes, as k/v row strides are at most 2^24 elements)
    const int nrec = (nvalid - 1) * (int)stride * 2 + 2 * D;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)tb, (short)0, nrec, 0x00020000);
    // LDS destination: the wave's share of the stage.  The base goes through
    // an empty asm so that the per-stage addresses are formed here (one
    // scalar add) instead of being hoisted into registers for the kernel.
    unsigned lb = smem_lds + (unsigned)wv * NL * 1024;
    asm volatile("" : "+s"(lb));
    char* dst = (char*)&smem[0][0] + (lb - smem_lds) + decltype(STAGE)::value * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + i * 1024), 16, goff[i], 0, 0, 0);
  };

  // Per-lane LDS byte addresses inside a K or V tile (rows of 2D bytes).
  // K, A operand of S^T for the 32-key unit at row 32 h of the tile: row
  // 32 h + lr, logical slot 2c + lg: kaddr[c] + (K stage) + 64 D h.
  unsigned kaddr[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) kaddr[c] = smem_lds + lr * 2 * D + 16 * swz<SLOTS>(lr, 2 * c + lg);
  // V, transposing reads for the unit at row 32 h, 16-key group hh, second 8
  // rows (+8): source lane j = lane % 16 supplies row 32 h + 16 hh + 8 half +
  // 4 (lane / 32) + j / 4 and the 8 bytes at channel 32 db + 16 ((lane / 16) % 2)
  // + 4 (j % 4), i.e. logical slot 4 db + 2 ((lane / 16) % 2) + (j % 4) / 2,
  // byte 8 (j % 2): voff[half][db] + (V stage) + 2D (32 h + 16 hh).
  const int vj = lane & 15, ve = vj >> 2, vc = vj & 3, vgrp = lane >> 4;
  const int vx = 2 * (vgrp & 1) + (vc >> 1);
  unsigned voff[2][DB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 4 * lg + ve + 8 * half;
      voff[half][db] = smem_lds + 4 * TILE_BYTES + r * 2 * D + 16 * swz<SLOTS>(r, 4 * db + vx) + 8 * (vc & 1);
    }

  // ---- schedule ----------------------------------------------------------
  // The workgroup's key tiles c_0 .. c_{n-1} (ring order, causal tiles past
  // the last query dropped; 64 keys each) are processed as 32-key units
  // u = 2t + h (half h of tile t).  Every wave runs the same software
  // pipeline, one step per unit: step u issues the MFMAs of
  //   S(u+1) = K(u+1) Q^T   and   O^T += V(u-1)^T P(u-1)^T
  // interleaved with the vector work of the softmax of S(u) (P(u) =
  // exp2(S c - m), row sum), which depends on neither; the mask of a tile
  // that needs one precedes the step, a redo of the unit follows it.  Two waves
  // share each SIMD, so both the matrix cores and the vector ALUs are fed by
  // two instruction streams.  The K fragments of unit u+1 are read in the
  // second half of step u-1, the V^T fragments of unit u-1 in the first half
  // of step u.  One barrier per tile: iteration t (units 2t, 2t+1) starts by
  // publishing K(c_{t+1}) and V(c_t) (loaded two iterations earlier) and then
  // issues the loads of K(c_{t+3}) and V(c_{t+2}).  Tile c_t sits in K and V
  // stage t % 4; the loop body covers four iterations, so every LDS offset
  // of a read is an immediate on a per-lane base fixed for the kernel.
  int n = 0;
  for (int s = 0; s < nsteps; ++s) n += step_tiles(s);

  if (n > 0) {  // workgroup-uniform
    const int64_t roff = a.ring ? 0 : a.kv_off;  // key position - row in k/v
    const int64_t q0w = qpos0 + qrow_w;          // the wave's first query position
    const int64_t kstep = (int64_t)BN * a.k_ss * 2, vstep = (int64_t)BN * a.v_ss * 2;
    // Cursor over the tiles: loop step cs, tile cu of its cnt tiles, the
    // tile's key position relative to the wave's first query (saturated at
    // +-2^30: a tile that far before the queries is fully visible, one that
    // far after them is never walked under causal masking, and the position
    // is not used without it; a block holds at most 2^29 keys, so the
    // position stays on its side of zero), keys left in the block from it
    // on, K and V addresses of its first row.
    constexpr int kRelSat = 1 << 30;
    int cs = 0, cu = 0, cnt = 0, crel = 0, cleft = 0;
    const char* cka = kbase;
    const char* cva = vbase;
    auto cur_set = [&]() {
      cu = 0;
      cnt = step_tiles(cs);
      const int64_t kv = step_kv_off(cs), rel = kv - q0w;
      crel = rel < -kRelSat ? -kRelSat : (rel > kRelSat ? kRelSat : (int)rel);
      cleft = (int)step_keys(cs);
      cka = kbase + (kv - roff) * a.k_ss * 2;
      cva = vbase + (kv - roff) * a.v_ss * 2;
    };
    while (step_tiles(cs) == 0) ++cs;
    cur_set();
    // Descriptors of tiles t .. t+3 (relative key position, valid rows, K and
    // V addresses, whether the tile needs a mask) in slots t % 4 .. (t + 3) % 4.  Past the last tile a slot
    // keeps the descriptor it held (an earlier tile): the loads made with it
    // land in stages nobody reads, which keeps the loads unconditional.
    int rem = n;
    int drel[4], dv[4];  // dv: valid rows, + 128 if the tile needs a mask
    const char* dka[4];
    const char* dva[4];
    auto fill = [&](auto SLOT) __attribute__((always_inline)) {
      constexpr int j = decltype(SLOT)::value;
      if (rem > 0) {
        drel[j] = crel;
        const int nv = cleft < BN ? cleft : BN;
        dv[j] = nv + (ra_plan_tile_masked<int>(crel, nv, BN, a.causal) ? 128 : 0);
        dka[j] = cka;
        dva[j] = cva;
        if (--rem > 0) {
          if (++cu < cnt) {
            crel += BN;
            cleft -= BN;
            cka += kstep;
            cva += vstep;
          } else {
            do {
              ++cs;
            } while (cs < nsteps && step_tiles(cs) == 0);
            if (cs < nsteps) cur_set();
          }
        }
      }
    };
    auto load_k = [&](auto ST) __attribute__((always_inline)) {
      constexpr int j = decltype(ST)::value;
      issue(dka[j], a.k_ss, koffg, dv[j] & 127, ST);
    };
    auto load_v = [&](auto ST) __attribute__((always_inline)) {
      constexpr int j = decltype(ST)::value;
      issue(dva[j], a.v_ss, voffg, dv[j] & 127, std::integral_constant<int, 4 + j>{});
    };

    f32x16 sacc[2];           // S^T of units with even / odd index
    bf16x8 pf[2][2];          // P^T of units with even / odd index, per 16-key group
    bf16x8 kf[KC];            // K fragments of the next S^T
    u32x2 vlo[2][DB], vhi[2][DB];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sacc[i] = f32x16{};
      pf[i][0] = pf[i][1] = bf16x8{};
    }

    // ---- LDS reads: inline asm with explicit waits that carry the registers
    // they guarantee (the compiler's waits would order them behind the
    // in-flight direct loads: it cannot prove they do not alias).  LDS reads
    // complete in order; scalar loads only make a wait stricter.  KO / VO:
    // byte offset of the unit in the K / V region (stage * tile + half * 64D),
    // an immediate; rt: a run-time offset added to the bases (0 in the loop).
    auto kread = [&kf, &kaddr](auto KO) __attribute__((always_inline)) {
      constexpr unsigned ko = decltype(KO)::value;
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[c]) : "v"(kaddr[c]), "i"(ko));
    };
    // wait until at most N LDS reads are in flight; the K fragments are older
    auto kwait0 = [&kf]() __attribute__((always_inline)) {
      if constexpr (KC == 8)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]), "+v"(kf[4]),
                     "+v"(kf[5]), "+v"(kf[6]), "+v"(kf[7]));
      else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]));
    };
    // V^T fragments, 16-key group HH of the unit at offset VO (+ rt).
    auto vread = [&vlo, &vhi, &voff](auto HH, auto VO, unsigned rt) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
      constexpr unsigned vo = decltype(VO)::value + (unsigned)hh * 32 * D;
#pragma unroll
      for (int x = 0; x < DB; ++x) {
        const unsigned a0 = voff[0][x] + rt, a1 = voff[1][x] + rt;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vlo[hh][x]) : "v"(a0), "i"(vo));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vhi[hh][x]) : "v"(a1), "i"(vo));
      }
    };
    // group 0 done (group 1 and the next K reads may be in flight), group 1
    // done (the next K reads may be in flight)
    auto vwait0 = [&vlo, &vhi]() __attribute__((always_inline)) {
      if constexpr (D == 128)
        asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(vlo[0][0]), "+v"(vhi[0][0]), "+v"(vlo[0][1]), "+v"(vhi[0][1]),
                     "+v"(vlo[0][2]), "+v"(vhi[0][2]), "+v"(vlo[0][3]), "+v"(vhi[0][3]));
      else
        asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(vlo[0][0]), "+v"(vhi[0][0]), "+v"(vlo[0][1]), "+v"(vhi[0][1]));
    };
    auto vwait1 = [&vlo, &vhi](auto KN) __attribute__((always_inline)) {
      constexpr int pend = decltype(KN)::value ? KC : 0;  // K reads issued after group 1
      if constexpr (D == 128)
        asm volatile("s_waitcnt lgkmcnt(%8)" : "+v"(vlo[1][0]), "+v"(vhi[1][0]), "+v"(vlo[1][1]), "+v"(vhi[1][1]),
                     "+v"(vlo[1][2]), "+v"(vhi[1][2]), "+v"(vlo[1][3]), "+v"(vhi[1][3]) : "n"(pend));
      else
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(vlo[1][0]), "+v"(vhi[1][0]), "+v"(vlo[1][1]), "+v"(vhi[1][1])
                     : "n"(pend));
    };

    // Softmax of the unit whose S^T is in sacc[x], at key position k0 with
    // nvalid valid keys.  Mask (a rare branch before the step's region): keys
    // kvi < lim of the unit are visible to this lane's query: lim = valid keys,
    // cut at the query's own position under causal masking (0 when the whole
    // unit lies after it: p = 0).  The key index of register r is
    // 8 (r / 4) + (r % 4) + 4 lg.
    auto sm_mask = [&](int x, int64_t k0, int nvalid) __attribute__((always_inline)) {
      // every key valid and, under causal masking, at or before the wave's
      // first query: nothing to mask (rows past nq are never stored)
      if (__builtin_expect(ra_plan_tile_masked<int64_t>(k0 - q0w, nvalid, 32, a.causal), 0)) {
        const int lim = (int)ra_plan_visible_prefix(q0w + lr, k0, nvalid, a.causal) - 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[x][r] = (8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : sacc[x][r];
      }
    };
    // Softmax of unit u against the running max m2 (log2 units) as it
    // stands: p = exp2(s c - m2), two keys per slot of the pipeline step, and
    // the fp32 row sum (only the MFMA operand is rounded to bf16: rows with
    // few visible keys would otherwise carry the 2^-9 rounding of one term
    // into l and the LSE).  The row max is not computed on this path.  When a
    // lane's sum of p exceeds kRedoSum or is not finite (m2 still -inf, or
    // an overflow), the whole unit is redone after the step against its
    // exact row max, which becomes m2 (sm_fix).  So m2 moves only on a redo,
    // every p stays at most kRedoSum, and o, l and m2 always agree: the
    // result does not depend on which max was used.  Each step pins its
    // results with an empty asm statement (the compiler would otherwise sink
    // the arithmetic towards its consumers, out of the region it is meant to
    // overlap with).
    float sm_ps[4], sm_tot = 0.f;
    auto sm_step = [&](auto X, auto ST) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, k = decltype(ST)::value;
      const f32x16& s = sacc[x];
      const float p0 = fast_exp2(fmaf(s[2 * k], a.c, -m2));
      const float p1 = fast_exp2(fmaf(s[2 * k + 1], a.c, -m2));
      if constexpr (k < 4) sm_ps[k] = p0 + p1;
      else sm_ps[k - 4] += p0 + p1;
      pf[x][k >> 2][2 * (k & 3)] = (__bf16)p0;
      pf[x][k >> 2][2 * (k & 3) + 1] = (__bf16)p1;
      asm volatile("" : "+v"(sm_ps[k & 3]), "+v"(pf[x][k >> 2]));
      if constexpr (k == 7) {
        sm_tot = (sm_ps[0] + sm_ps[1]) + (sm_ps[2] + sm_ps[3]);
        asm volatile("" : "+v"(sm_tot));
      }
    };
    // After the step: redo the unit if any lane asks for it, then add its
    // row sum.  The redo moves m2 to the exact row max, rescales o and l by
    // alpha = exp2(m2_old - m2_new) (0 when m2 was -inf) and recomputes p
    // (0 for rows with no visible key yet).
    auto sm_fix = [&](auto X) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(sm_tot <= kRedoSum)) != 0, 0)) {
        const f32x16& s = sacc[x];
        float mx = vmax3(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], s[5]), vmax3(s[6], s[7], s[8]));
        mx = vmax3(mx, vmax3(s[9], s[10], s[11]), vmax3(s[12], s[13], s[14]));
        mx = vmax3(mx, s[15], s[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float tm = vmax3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1])) * a.c;
        const bool up = tm > m2;
        const float alpha = up ? fast_exp2(m2 - tm) : 1.f;
        m2 = up ? tm : m2;
        const float muse = m2 == -INFINITY ? 0.f : m2;
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float p0 = fast_exp2(fmaf(s[2 * k], a.c, -muse));
          const float p1 = fast_exp2(fmaf(s[2 * k + 1], a.c, -muse));
          tot += p0 + p1;
          pf[x][k >> 2][2 * (k & 3)] = (__bf16)p0;
          pf[x][k >> 2][2 * (k & 3) + 1] = (__bf16)p1;
          asm volatile("" : "+v"(pf[x][k >> 2]), "+v"(tot));
        }
        sm_tot = tot;
        lsum *= alpha;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
      }
      lsum += sm_tot;
    };

    // MFMA m of a step: m < KC: step c = m of S^T(u+1) into sacc[XN]; else
    // O^T += V^T P^T(u-1) for 16-key group hh and channel block db, P from
    // pf[XP].  (Their results are not pinned: an instruction that reads an
    // MFMA result waits for the MFMA to finish.)
    auto mma = [&](auto XN, auto XP, auto M) __attribute__((always_inline)) {
      constexpr int xn = decltype(XN)::value, xp = decltype(XP)::value, m = decltype(M)::value;
      if constexpr (m < KC) {
        if constexpr (m == 0)
          sacc[xn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], f32x16{}, 0, 0, 0);
        else
          sacc[xn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m], qf[m], sacc[xn], 0, 0, 0);
      } else {
        constexpr int hh = (m - KC) / DB, db = (m - KC) % DB;
        const u32x4 w = {vlo[hh][db][0], vlo[hh][db][1], vhi[hh][db][0], vhi[hh][db][1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[xp][hh], o[db], 0, 0, 0);
      }
    };
    constexpr int MPS = (KC + 2 * DB) / 8;  // MFMAs per slot
    static_assert(MPS * 8 == KC + 2 * DB, "eight slots per step");
    const std::integral_constant<int, 0> X0;
    const std::integral_constant<int, 1> X1;
    const std::integral_constant<int, 0> H0;
    const std::integral_constant<int, 1> H1;
    // Pipeline step for unit u (S^T(u) in sacc[X], P(u-1) in pf[1-X]): SN: the
    // next unit exists (its K fragments are in kf: S^T(u+1) into sacc[1-X]);
    // PV: the previous unit exists (its V^T at offset VO + vrt); SM: unit u
    // exists (softmax); KN: read the K fragments of unit u+2 (offset KO) in
    // the second half; load(): this step's tile load, issued in slot 2.
    // Eight slots of one softmax step and MPS MFMAs each, kept in order by
    // scheduling barriers: S^T(u+1) in slots 0-3 (its K fragments arrived
    // during the previous step), O^T in slots 4-7 (the V^T reads issued in
    // slots 0 and 1 land meanwhile).
    auto step = [&](auto X, auto SN, auto PV, auto SM, auto KN, auto VO, unsigned vrt, auto KO, auto load)
        __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value;
      constexpr bool sn = decltype(SN)::value, pv = decltype(PV)::value, sm = decltype(SM)::value;
      constexpr bool kn = decltype(KN)::value;
      static_for<0, 8>([&](auto SL) {
        constexpr int sl = decltype(SL)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (sl == 0) {
          if constexpr (sn) kwait0();
          if constexpr (pv) vread(H0, VO, vrt);
        }
        if constexpr (sl == 1 && pv) vread(H1, VO, vrt);
        if constexpr (sl == 4) {
          if constexpr (pv) vwait0();
          if constexpr (kn) kread(KO);
        }
        if constexpr (sl == 6 && pv) vwait1(KN);  // the K reads for the next step (if any) are younger
        if constexpr (sl == 2) load();
        if constexpr (sm) sm_step(X, SL);
        static_for<sl * MPS, (sl + 1) * MPS>([&](auto M) {
          constexpr int m = decltype(M)::value;
          if constexpr (m < KC) {
            if constexpr (sn) mma(std::integral_constant<int, 1 - x>{}, std::integral_constant<int, 1 - x>{}, M);
          } else if constexpr (pv) {
            mma(std::integral_constant<int, 1 - x>{}, std::integral_constant<int, 1 - x>{}, M);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (sm) sm_fix(X);
    };
    auto half_valid = [](int nv, int hf) { return ra_plan_half_valid(nv, hf, 32); };
    const std::true_type T;
    const std::false_type F;
    // byte offset of half H of the tile in stage S (K and V regions alike)
    auto uoff = [](auto S, auto H) {
      return std::integral_constant<unsigned, (unsigned)decltype(S)::value * TILE_BYTES +
                                                  (unsigned)decltype(H)::value * 64 * D>{};
    };
    using std::integral_constant;

    // Prologue: descriptors of c_0..3; K(c_0..2), V(c_0..1); V stage 3
    // cleared (the first step's P V reads it with P = 0); S^T of unit 0; K
    // fragments of unit 1.
    fill(integral_constant<int, 0>{});
#pragma unroll
    for (int j = 1; j < 4; ++j) drel[j] = drel[0], dv[j] = dv[0], dka[j] = dka[0], dva[j] = dva[0];
    fill(integral_constant<int, 1>{});
    fill(integral_constant<int, 2>{});
    fill(integral_constant<int, 3>{});
    load_k(integral_constant<int, 0>{});
    load_k(integral_constant<int, 1>{});
    load_k(integral_constant<int, 2>{});
    load_v(integral_constant<int, 0>{});
    load_v(integral_constant<int, 1>{});
    {
      constexpr int per = TILE_BYTES / (NW * 64 * 16);  // 16-byte stores per lane
#pragma unroll
      for (int i = 0; i < per; ++i) *(u32x4*)(&smem[7][0] + (i * NW * 64 + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    kread(uoff(integral_constant<int, 0>{}, H0));
    kwait0();
#pragma unroll
    for (int c = 0; c < KC; ++c)
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[c], c == 0 ? f32x16{} : sacc[0], 0, 0, 0);
    kread(uoff(integral_constant<int, 0>{}, H1));  // unit 1 (waited for at the first step)

    // Iteration head: the barrier that publishes K(c_{t+1}) and V(c_t): all
    // loads but those of the previous iteration (K(c_{t+2}), V(c_{t+1})) are
    // complete.
    auto head = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NL) : "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // Every iteration runs the same two steps (a second variant of a step in
    // the loop costs registers everywhere): at t = 0 the P V of the
    // nonexistent unit -1 adds P = 0 times the zeros of V stage 3; in the
    // last iteration S^T of the nonexistent unit 2n and the K reads past the
    // end fill registers that are never used (stale but in-bounds LDS).  Unit
    // 2t has its S^T in sacc[0], unit 2t+1 in sacc[1].
    auto iter = [&](auto J) __attribute__((always_inline)) {  // iteration t, J = t % 4
      constexpr int j = decltype(J)::value;
      const integral_constant<int, j> SJ;
      const integral_constant<int, (j + 1) & 3> SJ1;
      const integral_constant<int, (j + 2) & 3> SJ2;
      const integral_constant<int, (j + 3) & 3> SJ3;
      const bool mt = dv[j] >= 128;
      if (__builtin_expect(mt, 0)) sm_mask(0, q0w + drel[j], half_valid(dv[j] & 127, 0));
      // unit 2t: P V of unit 2t-1 (c_{t-1}, half 1), K of unit 2t+2 (c_{t+1}, half 0), load K(c_{t+3})
      step(X0, T, T, T, T, uoff(SJ3, H1), 0u, uoff(SJ1, H0), [&]() __attribute__((always_inline)) { load_k(SJ3); });
      if (__builtin_expect(mt, 0)) sm_mask(1, q0w + drel[j] + 32, half_valid(dv[j] & 127, 1));
      // unit 2t+1: P V of unit 2t (c_t, half 0), K of unit 2t+3 (c_{t+1}, half 1), load V(c_{t+2})
      step(X1, T, T, T, T, uoff(SJ, H0), 0u, uoff(SJ1, H1), [&]() __attribute__((always_inline)) { load_v(SJ2); });
      fill(SJ);  // slot of c_t now holds c_{t+4}
    };
    int t = 0;
    for (;;) {
      iter(integral_constant<int, 0>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 1>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 2>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 3>{});
      if (++t == n) break;
      head();
    }
    // drain: O^T += V^T P^T of the last unit (half 1 of c_{n-1}, P in pf[1])
    step(X0, F, T, F, F, uoff(integral_constant<int, 0>{}, H1), (unsigned)((n - 1) & 3) * TILE_BYTES,
         uoff(integral_constant<int, 0>{}, H0), []() {});
    // the last iterations' loads (into stages nobody reads) land before the
    // workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    for (int db = 0; db < DB; ++db)
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
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 x = {(__bf16)(o[db][4 * j] * inv), (__bf16)(o[db][4 * j + 1] * inv),
                      (__bf16)(o[db][4 * j + 2] * inv), (__bf16)(o[db][4 * j + 3] * inv)};
          *(bf16x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
        }
    } else {
      float* op = (float*)a.o + base;
#pragma unroll
      for (int db = 0; db < DB; ++db)
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

// bf16 path with 64 query rows per wave (attn_bf16_w64_kernel): one
// workgroup = 4 waves = 256 query rows, one wave per SIMD.  Every K and V^T
// fragment a wave reads from LDS feeds the MFMAs of two 32-row blocks (rb =
// 0, 1), so a key tile costs half the LDS reads and half the tile
// bookkeeping per MFMA of the 32-rows-per-wave form above.  The price is the
// register file: the output accumulators of both row blocks (2 x D/32 x 16
// fp32) live in AGPRs, pinned there by the P V products being inline-asm
// MFMAs, and a SIMD's matrix core is fed by one instruction stream, so each
// pipeline step alternates single MFMAs with short runs of the softmax's
// vector work (16 slots of two MFMAs per 32-key unit).  Everything else --
// tile walk, direct loads, swizzle, lazy softmax with exact redo, epilogue --
// is the form above, per row block.

// The MFMAs of attn_bf16_w64_kernel, inline asm so that the operands sit in
// the register file the kernel needs them in (the builtins leave that to the
// compiler, which then runs out of VGPRs and copies between the files).
// The compiler does not see the wait states around inline-asm MFMAs (gfx950,
// as the compiler itself spaces its own MFMAs: 2 after a vector write of an
// operand, none between dependent products, 12 before a vector read of a
// result):
//   - after a vector write of an operand: the P V product's leading s_nop 1
//     (its A operand may have just been assembled by vector moves, its C may
//     have just been rescaled); the S^T product's operands come from LDS
//     reads (waited for) and from the Q fragments, written once before the
//     first product, which has its own s_nop;
//   - before a vector read of a result: the kernel's drains (16 wait
//     states), and otherwise whole pipeline slots between the write and the
//     read.
// S^T (keys x queries) = K Q^T, k-step 0 (C = 0) and later k-steps; the
// accumulator in VGPRs, the Q fragment (B) in AGPRs.
__device__ __forceinline__ void mfma_s_first(f32x16& c, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_s_next(f32x16& c, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(k), "a"(q));
}
// O^T += V^T P^T with the accumulator pinned to AGPRs.
__device__ __forceinline__ void mfma_pv(f32x16& c, const bf16x8& A, const bf16x8& B) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(A), "v"(B));
}

template <int D>
__global__ void __launch_bounds__(256, 1) attn_bf16_w64_kernel(RaAttnArgs a) {
  constexpr int NW = 4, RB = 2, BM = NW * 32 * RB, BN = RA_BF16_BN;
  constexpr int SLOTS = D / 8;                 // 16-byte slots per row
  constexpr int TILE_BYTES = BN * D * 2;       // one K or V tile
  constexpr int NL = TILE_BYTES / 1024 / NW;   // 1 KiB direct loads per wave per tile
  constexpr int KC = D / 16;                   // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                   // 32-channel blocks of O^T
  static_assert(NL * 1024 * NW == TILE_BYTES, "tile split");
  static_assert(BM == RA_BF16_BM && BN == 64, "64-key tiles, processed as two 32-key units");
  // [0] .. [3]: K stages; [4] .. [7]: V stages (tile c_t in K and V stage t % 4)
  __shared__ __attribute__((aligned(1024))) char smem[8][TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep per-wave values in SGPRs
  const int lr = lane & 31, lg = lane >> 5;

  // query tiles: nqt_c per chunk of nqc rows (one chunk unless the share is split)
  const int nqc = a.nsplit == 2 ? (int)a.qc : a.nq;
  const int nqt_c = (nqc + BM - 1) / BM;
  const int nqt = (a.nsplit == 2 ? 2 : 1) * nqt_c;
  int hb, qt;  // later query tiles see more keys under causal masking: they start first
  ra_plan_head_tile(ra_plan_xcd_remap(blockIdx.x, gridDim.x, nqt), gridDim.x, nqt, a.causal, &hb, &qt);
  const int h = hb % a.Hq, b = hb / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int chunk = qt / nqt_c;
  const int64_t qpos0 = chunk ? a.q_off2 : a.q_off;  // global position of the chunk's first row
  const int rank_e = chunk ? a.rank2 : a.rank;        // its ring order

  const int qrow_wg = (qt - chunk * nqt_c) * BM;      // rows within the chunk
  const int qrow_w = qrow_wg + wave * 32 * RB;        // the wave's first row
  int my_q[RB];                                       // local rows (q, o, lse, state) of the lane
  bool q_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_q[rb] = chunk * nqc + qrow_w + 32 * rb + lr;
    q_ok[rb] = qrow_w + 32 * rb + lr < nqc;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[my_q[rb]][16c + 8lg .. +7].
  bf16x8 qf[RB][KC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)(q_ok[rb] ? my_q[rb] : 0) * a.q_ss +
                       (int64_t)h * a.q_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_ok[rb]) w = *(const u32x4*)(qp + 16 * c);
      qf[rb][c] = __builtin_bit_cast(bf16x8, w);
      asm volatile("" : "+a"(qf[rb][c]));  // from here on the fragment lives in AGPRs
    }
  }

  // Running state per row block.  o[rb][db][r] = O^T[32db + 8(r/4) + 4lg +
  // r%4][my_q[rb]] (unnormalised, in AGPRs); m2 = running max of s * c (log2
  // units); lsum = this lane's half of the row sum.
  f32x16 o[RB][DB];
  float m2[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m2[rb] = -INFINITY;
    lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x16{};
    if (a.state_in && q_ok[rb]) {
      const float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q[rb] * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 x = *(const f32x4*)(op + 32 * db + 8 * j + 4 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][db][4 * j + i] = x[i];
        }
      const float mv = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q[rb] * a.m_ss];
      const float lv = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q[rb] * a.l_ss];
      m2[rb] = mv * kLog2e;  // -inf stays -inf
      lsum[rb] = lg == 0 ? lv : 0.f;
    }
  }
  // The accumulators are read by vector code (a redo, the epilogue) only
  // after this: 16 wait states after the last MFMA that wrote them.
  auto ofrag_drain = [&o]() __attribute__((always_inline)) {
    if constexpr (DB == 4)
      asm volatile("s_nop 7\n\ts_nop 7"
                   : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                     "+a"(o[1][2]), "+a"(o[1][3]));
    else
      asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
  };

  const int64_t q0_wg = qpos0 + qrow_wg;
  const int nq_wg = min(BM, nqc - qrow_wg);
  const int nsteps = a.ring ? a.P : 1;
  // Block order as in attn_bf16_kernel: ring order with the rank's own block
  // (ring step 0) folded last.
  auto step_kv_off = [&](int s) -> int64_t {
    return a.ring ? (int64_t)ra_plan_ring_block32(a.P, rank_e, (s + 1) % a.P) * a.nkv : a.kv_off;
  };
  auto step_keys = [&](int s) -> int64_t {
    const int64_t n = a.kv_end - step_kv_off(s);
    return n < 0 ? 0 : (n < a.nkv ? n : a.nkv);
  };
  auto step_tiles = [&](int s) -> int {
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, step_kv_off(s), step_keys(s), a.causal, BN);
  };

  // Direct loads, as in attn_bf16_kernel, with the tile split over 4 waves.
  const char* kbase = (const char*)a.k + 2 * ((int64_t)b * a.k_sb + (int64_t)hk * a.k_sh);
  const char* vbase = (const char*)a.v + 2 * ((int64_t)b * a.v_sb + (int64_t)hk * a.v_sh);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto gslot = [&](int i, int& r) -> unsigned {
    const int ls = (wv * NL + i) * 64 + lane;
    r = ls / SLOTS;
    return 16u * (unsigned)swz<SLOTS>(r, ls % SLOTS);
  };
  unsigned koffg[NL], voffg[NL];  // row strides of k and v: at most 2^24 elements
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    int r;
    const unsigned sl = gslot(i, r);
    koffg[i] = (unsigned)r * (unsigned)a.k_ss * 2u + sl;
    voffg[i] = (unsigned)r * (unsigned)a.v_ss * 2u + sl;
  }
  const unsigned smem_lds = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)&smem[0][0]);
  // Chunk CHUNK (1 KiB, one instruction) of the wave's share of a tile:
  // the loads of a tile are spread over consecutive pipeline slots.
  auto issue = [&](const char* tb, int64_t stride, const unsigned* goff, int nvalid, auto STAGE, auto CHUNK)
      __attribute__((always_inline)) {
    const int nrec = (nvalid - 1) * (int)stride * 2 + 2 * D;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)tb, (short)0, nrec, 0x00020000);
    unsigned lb = smem_lds + (unsigned)wv * NL * 1024;
    asm volatile("" : "+s"(lb));
    char* dst = (char*)&smem[0][0] + (lb - smem_lds) + decltype(STAGE)::value * TILE_BYTES;
    constexpr int i = decltype(CHUNK)::value;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + i * 1024), 16, goff[i], 0, 0, 0);
  };

  unsigned kaddr[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) kaddr[c] = smem_lds + lr * 2 * D + 16 * swz<SLOTS>(lr, 2 * c + lg);
  const int vj = lane & 15, ve = vj >> 2, vc = vj & 3, vgrp = lane >> 4;
  const int vx = 2 * (vgrp & 1) + (vc >> 1);
  unsigned voff[2][DB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 4 * lg + ve + 8 * half;
      voff[half][db] = smem_lds + 4 * TILE_BYTES + r * 2 * D + 16 * swz<SLOTS>(r, 4 * db + vx) + 8 * (vc & 1);
    }

  int n = 0;
  for (int s = 0; s < nsteps; ++s) n += step_tiles(s);

  if (n > 0) {  // workgroup-uniform
    const int64_t roff = a.ring ? 0 : a.kv_off;
    const int64_t q0w = qpos0 + qrow_w;          // the wave's first query position
    const int64_t kstep = (int64_t)BN * a.k_ss * 2, vstep = (int64_t)BN * a.v_ss * 2;
    constexpr int kRelSat = 1 << 30;
    int cs = 0, cu = 0, cnt = 0, crel = 0, cleft = 0;
    const char* cka = kbase;
    const char* cva = vbase;
    auto cur_set = [&]() {
      cu = 0;
      cnt = step_tiles(cs);
      const int64_t kv = step_kv_off(cs), rel = kv - q0w;
      crel = rel < -kRelSat ? -kRelSat : (rel > kRelSat ? kRelSat : (int)rel);
      cleft = (int)step_keys(cs);
      cka = kbase + (kv - roff) * a.k_ss * 2;
      cva = vbase + (kv - roff) * a.v_ss * 2;
    };
    while (step_tiles(cs) == 0) ++cs;
    cur_set();
    int rem = n;
    int drel[4], dv[4];  // dv: valid rows, + 128 if the tile needs a mask for some row of the wave
    const char* dka[4];
    const char* dva[4];
    auto fill = [&](auto SLOT) __attribute__((always_inline)) {
      constexpr int j = decltype(SLOT)::value;
      if (rem > 0) {
        drel[j] = crel;
        const int nv = cleft < BN ? cleft : BN;
        dv[j] = nv + (ra_plan_tile_masked<int>(crel, nv, BN, a.causal) ? 128 : 0);
        dka[j] = cka;
        dva[j] = cva;
        if (--rem > 0) {
          if (++cu < cnt) {
            crel += BN;
            cleft -= BN;
            cka += kstep;
            cva += vstep;
          } else {
            do {
              ++cs;
            } while (cs < nsteps && step_tiles(cs) == 0);
            if (cs < nsteps) cur_set();
          }
        }
      }
    };
    auto load_k = [&](auto ST, auto CH) __attribute__((always_inline)) {
      constexpr int j = decltype(ST)::value;
      issue(dka[j], a.k_ss, koffg, dv[j] & 127, ST, CH);
    };
    auto load_v = [&](auto ST, auto CH) __attribute__((always_inline)) {
      constexpr int j = decltype(ST)::value;
      issue(dva[j], a.v_ss, voffg, dv[j] & 127, std::integral_constant<int, 4 + j>{}, CH);
    };
    auto load_k_all = [&](auto ST) __attribute__((always_inline)) {
      static_for<0, NL>([&](auto CH) { load_k(ST, CH); });
    };
    auto load_v_all = [&](auto ST) __attribute__((always_inline)) {
      static_for<0, NL>([&](auto CH) { load_v(ST, CH); });
    };

    f32x16 sacc[2][RB];       // S^T of units with even / odd index, per row block
    bf16x8 pf[2][RB][2];      // P^T of units with even / odd index, per row block and 16-key group
    bf16x8 kf[KC];            // K fragments of the next S^T
    u32x2 vlo[2][DB], vhi[2][DB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        sacc[i][rb] = f32x16{};
        pf[i][rb][0] = pf[i][rb][1] = bf16x8{};
      }

    auto kread = [&kf, &kaddr](auto KO) __attribute__((always_inline)) {
      constexpr unsigned ko = decltype(KO)::value;
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[c]) : "v"(kaddr[c]), "i"(ko));
    };
    auto kwait0 = [&kf]() __attribute__((always_inline)) {
      if constexpr (KC == 8)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]), "+v"(kf[4]),
                     "+v"(kf[5]), "+v"(kf[6]), "+v"(kf[7]));
      else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]));
    };
    auto vread = [&vlo, &vhi, &voff](auto HH, auto VO, unsigned rt) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
      constexpr unsigned vo = decltype(VO)::value + (unsigned)hh * 32 * D;
#pragma unroll
      for (int x = 0; x < DB; ++x) {
        const unsigned a0 = voff[0][x] + rt, a1 = voff[1][x] + rt;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vlo[hh][x]) : "v"(a0), "i"(vo));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vhi[hh][x]) : "v"(a1), "i"(vo));
      }
    };
    auto vwait0 = [&vlo, &vhi]() __attribute__((always_inline)) {
      if constexpr (D == 128)
        asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(vlo[0][0]), "+v"(vhi[0][0]), "+v"(vlo[0][1]), "+v"(vhi[0][1]),
                     "+v"(vlo[0][2]), "+v"(vhi[0][2]), "+v"(vlo[0][3]), "+v"(vhi[0][3]));
      else
        asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(vlo[0][0]), "+v"(vhi[0][0]), "+v"(vlo[0][1]), "+v"(vhi[0][1]));
    };
    auto vwait1 = [&vlo, &vhi](auto KN) __attribute__((always_inline)) {
      constexpr int pend = decltype(KN)::value ? KC : 0;  // K reads issued after group 1
      if constexpr (D == 128)
        asm volatile("s_waitcnt lgkmcnt(%8)" : "+v"(vlo[1][0]), "+v"(vhi[1][0]), "+v"(vlo[1][1]), "+v"(vhi[1][1]),
                     "+v"(vlo[1][2]), "+v"(vhi[1][2]), "+v"(vlo[1][3]), "+v"(vhi[1][3]) : "n"(pend));
      else
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(vlo[1][0]), "+v"(vhi[1][0]), "+v"(vlo[1][1]), "+v"(vhi[1][1])
                     : "n"(pend));
    };

    // Mask of row block rb's unit (as attn_bf16_kernel's sm_mask, for the
    // wave's rows 32 rb ..).
    auto sm_mask = [&](int x, int rb, int64_t k0, int nvalid) __attribute__((always_inline)) {
      const int64_t q0r = q0w + 32 * rb;
      if (__builtin_expect(ra_plan_tile_masked<int64_t>(k0 - q0r, nvalid, 32, a.causal), 0)) {
        const int lim = (int)ra_plan_visible_prefix(q0r + lr, k0, nvalid, a.causal) - 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[x][rb][r] = (8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : sacc[x][rb][r];
      }
    };
    // Softmax sub-step j of a step (row block j % 2, keys 2k, 2k+1 of the
    // lane's 16 with k = j / 2), software-pipelined over the slots: the
    // exponent arguments of sub-step j are formed in the slot before, so a
    // slot runs the two exponentials (sm_a) under one MFMA and the sums, the
    // bf16 P and the next sub-step's arguments (sm_b) under the other.
    float sm_ps[RB][4], sm_tot[RB] = {0.f, 0.f}, sm_p[RB][2], sm_arg[2];
    auto sm_args = [&](auto X, auto J) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, j = decltype(J)::value, rb = j % 2, k = j / 2;
      const f32x16& s = sacc[x][rb];
      sm_arg[0] = fmaf(s[2 * k], a.c, -m2[rb]);
      sm_arg[1] = fmaf(s[2 * k + 1], a.c, -m2[rb]);
      asm volatile("" : "+v"(sm_arg[0]), "+v"(sm_arg[1]));
    };
    auto sm_a = [&](auto X, auto R, auto K) __attribute__((always_inline)) {
      constexpr int rb = decltype(R)::value;
      sm_p[rb][0] = fast_exp2(sm_arg[0]);
      sm_p[rb][1] = fast_exp2(sm_arg[1]);
      asm volatile("" : "+v"(sm_p[rb][0]), "+v"(sm_p[rb][1]));
    };
    auto sm_b = [&](auto X, auto R, auto K) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, rb = decltype(R)::value, k = decltype(K)::value;
      if constexpr (2 * k + rb + 1 < 16) sm_args(X, std::integral_constant<int, 2 * k + rb + 1>{});
      const float p0 = sm_p[rb][0], p1 = sm_p[rb][1];
      if constexpr (k < 4) sm_ps[rb][k] = p0 + p1;
      else sm_ps[rb][k - 4] += p0 + p1;
      pf[x][rb][k >> 2][2 * (k & 3)] = (__bf16)p0;
      pf[x][rb][k >> 2][2 * (k & 3) + 1] = (__bf16)p1;
      asm volatile("" : "+v"(sm_ps[rb][k & 3]), "+v"(pf[x][rb][k >> 2]));
      if constexpr (k == 7) {
        sm_tot[rb] = (sm_ps[rb][0] + sm_ps[rb][1]) + (sm_ps[rb][2] + sm_ps[rb][3]);
        asm volatile("" : "+v"(sm_tot[rb]));
      }
    };
    // After the step: redo a row block's unit if any lane asks for it (as
    // attn_bf16_kernel's sm_fix), then add its row sum.
    auto sm_fix = [&](auto X, auto R) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, rb = decltype(R)::value;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(sm_tot[rb] <= kRedoSum)) != 0, 0)) {
        const f32x16& s = sacc[x][rb];
        float mx = vmax3(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], s[5]), vmax3(s[6], s[7], s[8]));
        mx = vmax3(mx, vmax3(s[9], s[10], s[11]), vmax3(s[12], s[13], s[14]));
        mx = vmax3(mx, s[15], s[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float tm = vmax3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1])) * a.c;
        const bool up = tm > m2[rb];
        const float alpha = up ? fast_exp2(m2[rb] - tm) : 1.f;
        m2[rb] = up ? tm : m2[rb];
        const float muse = m2[rb] == -INFINITY ? 0.f : m2[rb];
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float p0 = fast_exp2(fmaf(s[2 * k], a.c, -muse));
          const float p1 = fast_exp2(fmaf(s[2 * k + 1], a.c, -muse));
          tot += p0 + p1;
          pf[x][rb][k >> 2][2 * (k & 3)] = (__bf16)p0;
          pf[x][rb][k >> 2][2 * (k & 3) + 1] = (__bf16)p1;
          asm volatile("" : "+v"(pf[x][rb][k >> 2]), "+v"(tot));
        }
        sm_tot[rb] = tot;
        lsum[rb] *= alpha;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
          ofrag_drain();
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
        }
      }
      lsum[rb] += sm_tot[rb];
    };

    // MFMAs of a step.  S^T(u+1) of row block rb, k-step c, into sacc[XN][rb];
    // O^T += V^T P^T(u-1) of row block rb for 16-key group hh and channel
    // block db, P from pf[XP][rb].
    auto mma_s = [&](auto XN, auto R, auto C) __attribute__((always_inline)) {
      constexpr int xn = decltype(XN)::value, rb = decltype(R)::value, c = decltype(C)::value;
      if constexpr (c == 0)
        mfma_s_first(sacc[xn][rb], kf[0], qf[rb][0]);
      else
        mfma_s_next(sacc[xn][rb], kf[c], qf[rb][c]);
    };
    auto mma_pv = [&](auto XP, auto R, auto M) __attribute__((always_inline)) {
      constexpr int xp = decltype(XP)::value, rb = decltype(R)::value, m = decltype(M)::value;
      constexpr int hh = m / DB, db = m % DB;
      const u32x4 w = {vlo[hh][db][0], vlo[hh][db][1], vhi[hh][db][0], vhi[hh][db][1]};
      mfma_pv(o[rb][db], __builtin_bit_cast(bf16x8, w), pf[xp][rb][hh]);
    };
    // Pipeline step for unit u (S^T(u) in sacc[X], P(u-1) in pf[1-X]), 16
    // slots.  Slots 0 .. KC-1 (two slots per k-step when D = 64): the S^T(u+1)
    // chains of both row blocks; the remaining slots: O^T += V^T P^T(u-1),
    // one MFMA per row block.  Each slot is MFMA, first half of a softmax
    // sub-step, MFMA, second half, in that order (scheduling barriers), so
    // the vector work issues while the matrix core runs.  The sixteen
    // softmax sub-steps (8 per row block) take one slot each.
    auto step = [&](auto X, auto SN, auto PV, auto SM, auto KN, auto VO, unsigned vrt, auto KO, auto load)
        __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value;
      constexpr bool sn = decltype(SN)::value, pv = decltype(PV)::value, sm = decltype(SM)::value;
      constexpr bool kn = decltype(KN)::value;
      constexpr int NS = 16;                  // slots
      constexpr int SSLOTS = 2 * KC;          // MFMAs of S^T(u+1), 2 per slot
      constexpr int SS = SSLOTS / 2;          // slots holding them
      static_assert(SS + RB * 2 * DB / 2 == NS || D == 64, "16 slots at D = 128");
      if constexpr (sm) sm_args(X, std::integral_constant<int, 0>{});
      static_for<0, NS>([&](auto SL) {
        constexpr int sl = decltype(SL)::value;
        // slot sl's two MFMAs: index j = 2 sl, 2 sl + 1 of the step's list
        // (S^T(u+1): j < SSLOTS, rb = j % 2, k-step j / 2; then P V: the
        // rest, rb = j % 2, m = (j - SSLOTS) / 2)
        auto mfma_j = [&](auto J) __attribute__((always_inline)) {
          constexpr int j = decltype(J)::value;
          if constexpr (j < SSLOTS) {
            if constexpr (sn) mma_s(std::integral_constant<int, 1 - x>{}, std::integral_constant<int, j % 2>{},
                                    std::integral_constant<int, j / 2>{});
          } else if constexpr (j - SSLOTS < RB * 2 * DB) {
            if constexpr (pv) mma_pv(std::integral_constant<int, 1 - x>{}, std::integral_constant<int, j % 2>{},
                                     std::integral_constant<int, (j - SSLOTS) / 2>{});
          }
        };
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (sl == 0) {
          if constexpr (sn) kwait0();
          if constexpr (pv) vread(std::integral_constant<int, 0>{}, VO, vrt);
        }
        if constexpr (sl == 1 && pv) vread(std::integral_constant<int, 1>{}, VO, vrt);
        if constexpr (sl == SS) {
          if constexpr (pv) vwait0();
          if constexpr (kn) kread(KO);
        }
        if constexpr (sl == SS + DB && pv) vwait1(KN);  // the K reads for the next step (if any) are younger
        if constexpr (sl >= 2 && sl < 2 + NL) load(std::integral_constant<int, sl - 2>{});
        __builtin_amdgcn_sched_barrier(0);
        mfma_j(std::integral_constant<int, 2 * sl>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (sm) sm_a(X, std::integral_constant<int, sl % 2>{}, std::integral_constant<int, sl / 2>{});
        __builtin_amdgcn_sched_barrier(0);
        mfma_j(std::integral_constant<int, 2 * sl + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (sm) sm_b(X, std::integral_constant<int, sl % 2>{}, std::integral_constant<int, sl / 2>{});
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (sm) {
        sm_fix(X, std::integral_constant<int, 0>{});
        sm_fix(X, std::integral_constant<int, 1>{});
      }
    };
    auto half_valid = [](int nv, int hf) { return ra_plan_half_valid(nv, hf, 32); };
    const std::true_type T;
    const std::false_type F;
    auto uoff = [](auto S, auto H) {
      return std::integral_constant<unsigned, (unsigned)decltype(S)::value * TILE_BYTES +
                                                  (unsigned)decltype(H)::value * 64 * D>{};
    };
    using std::integral_constant;
    const integral_constant<int, 0> X0, H0, R0;
    const integral_constant<int, 1> X1, H1, R1;

    // Prologue: descriptors of c_0..3; K(c_0..2), V(c_0..1); V stage 3
    // cleared (the first step's P V reads it with P = 0); S^T of unit 0 for
    // both row blocks; K fragments of unit 1.
    fill(integral_constant<int, 0>{});
#pragma unroll
    for (int j = 1; j < 4; ++j) drel[j] = drel[0], dv[j] = dv[0], dka[j] = dka[0], dva[j] = dva[0];
    fill(integral_constant<int, 1>{});
    fill(integral_constant<int, 2>{});
    fill(integral_constant<int, 3>{});
    load_k_all(integral_constant<int, 0>{});
    load_k_all(integral_constant<int, 1>{});
    load_k_all(integral_constant<int, 2>{});
    load_v_all(integral_constant<int, 0>{});
    load_v_all(integral_constant<int, 1>{});
    {
      constexpr int per = TILE_BYTES / (NW * 64 * 16);  // 16-byte stores per lane
#pragma unroll
      for (int i = 0; i < per; ++i) *(u32x4*)(&smem[7][0] + (i * NW * 64 + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    kread(uoff(integral_constant<int, 0>{}, H0));
    kwait0();
    asm volatile("s_nop 4" ::: "memory");  // the Q fragments' moves into AGPRs precede this
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mfma_s_first(sacc[0][rb], kf[0], qf[rb][0]);
#pragma unroll
    for (int c = 1; c < KC; ++c)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mfma_s_next(sacc[0][rb], kf[c], qf[rb][c]);
    // S^T of unit 0 is read by vector code (a mask) right at the first step
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sacc[0][0]), "+v"(sacc[0][1]));
    kread(uoff(integral_constant<int, 0>{}, H1));  // unit 1 (waited for at the first step)

    auto head = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NL) : "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    auto iter = [&](auto J) __attribute__((always_inline)) {  // iteration t, J = t % 4
      constexpr int j = decltype(J)::value;
      const integral_constant<int, j> SJ;
      const integral_constant<int, (j + 1) & 3> SJ1;
      const integral_constant<int, (j + 2) & 3> SJ2;
      const integral_constant<int, (j + 3) & 3> SJ3;
      const bool mt = dv[j] >= 128;
      if (__builtin_expect(mt, 0)) {
        sm_mask(0, 0, q0w + 0 + drel[j], half_valid(dv[j] & 127, 0));
        sm_mask(0, 1, q0w + drel[j], half_valid(dv[j] & 127, 0));
      }
      step(X0, T, T, T, T, uoff(SJ3, H1), 0u, uoff(SJ1, H0),
           [&](auto CH) __attribute__((always_inline)) { load_k(SJ3, CH); });
      if (__builtin_expect(mt, 0)) {
        sm_mask(1, 0, q0w + drel[j] + 32, half_valid(dv[j] & 127, 1));
        sm_mask(1, 1, q0w + drel[j] + 32, half_valid(dv[j] & 127, 1));
      }
      step(X1, T, T, T, T, uoff(SJ, H0), 0u, uoff(SJ1, H1),
           [&](auto CH) __attribute__((always_inline)) { load_v(SJ2, CH); });
      fill(SJ);
    };
    int t = 0;
    for (;;) {
      iter(integral_constant<int, 0>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 1>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 2>{});
      if (++t == n) break;
      head();
      iter(integral_constant<int, 3>{});
      if (++t == n) break;
      head();
    }
    step(X0, F, T, F, F, uoff(integral_constant<int, 0>{}, H1), (unsigned)((n - 1) & 3) * TILE_BYTES,
         uoff(integral_constant<int, 0>{}, H0), [](auto) {});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // Epilogue, per row block: the two halves of each row sum live in lanes
  // lr and lr + 32.
  ofrag_drain();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float ltot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum[rb]), __float_as_uint(lsum[rb]), false,
                                                       false);
      ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!q_ok[rb]) continue;
    if (a.out_state) {
      float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q[rb] * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 x = {o[rb][db][4 * j], o[rb][db][4 * j + 1], o[rb][db][4 * j + 2], o[rb][db][4 * j + 3]};
          *(f32x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
        }
      if (lg == 0) {
        a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q[rb] * a.m_ss] = m2[rb] * kLn2;
        a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q[rb] * a.l_ss] = ltot;
      }
    } else {
      const float inv = 1.f / ltot;
      const int64_t base = (int64_t)b * a.o_sb + (int64_t)my_q[rb] * a.o_ss + (int64_t)h * a.o_sh;
      if (a.o_bf16) {
        __bf16* op = (__bf16*)a.o + base;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x4 x = {(__bf16)(o[rb][db][4 * j] * inv), (__bf16)(o[rb][db][4 * j + 1] * inv),
                        (__bf16)(o[rb][db][4 * j + 2] * inv), (__bf16)(o[rb][db][4 * j + 3] * inv)};
            *(bf16x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
          }
      } else {
        float* op = (float*)a.o + base;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 x = {o[rb][db][4 * j] * inv, o[rb][db][4 * j + 1] * inv, o[rb][db][4 * j + 2] * inv,
                       o[rb][db][4 * j + 3] * inv};
            *(f32x4*)(op + 32 * db + 8 * j + 4 * lg) = x;
          }
      }
      if (lg == 0 && a.lse)
        a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)my_q[rb] * a.lse_ss] =
            (m2[rb] + __log2f(ltot)) * kLn2;
    }
  }
}

// fp32 path: fp32 FMA throughout (dot products, softmax, P V).  A workgroup
// takes 64 query rows; each row belongs to LPR = D / 64 lanes of one wave
// (lanes l and l ^ 32 when D = 128), each holding 64 channels of the row's
// Q and O in registers, so the partial dot products of a key meet in one
// cross-lane swap.  K and V tiles of 64 keys are staged in LDS and read by
// all lanes of a half at the same address (broadcast).  The online softmax
// runs over chunks of 16 keys held in registers: chunk max, rescale of O
// and l when it grows, exponentials, O += p V.
template <int D>
__global__ void __launch_bounds__(64 * (D / 64)) attn_f32_kernel(RaAttnArgs a) {
  constexpr int BM = RA_F32_BM, BN = RA_F32_BN, CH = 16;
  constexpr int LPR = D / 64, DL = D / LPR;  // lanes per row, channels per lane
  constexpr int NT = 64 * LPR;               // threads
  static_assert(DL == 64 && BM == 64, "64 channels per lane, 64 rows per workgroup");
  __shared__ __attribute__((aligned(16))) float Ks[BN * D];
  __shared__ __attribute__((aligned(16))) float Vs[BN * D];
  const int tid = threadIdx.x;
  // row of the workgroup and channel half: rows 32 w .. 32 w + 31 in wave w
  // when a row takes two lanes (l, l ^ 32), else row = lane
  const int lrow = LPR == 2 ? (tid >> 6) * 32 + (tid & 31) : tid;
  const int half = LPR == 2 ? (tid >> 5) & 1 : 0;
  const int c0 = half * DL;
  const int nqc = a.nsplit == 2 ? (int)a.qc : a.nq;  // rows per chunk
  const int nqt_c = (nqc + BM - 1) / BM;
  const int nqt = (a.nsplit == 2 ? 2 : 1) * nqt_c;
  const int qt = blockIdx.x % nqt;
  const int hb = blockIdx.x / nqt;
  const int h = hb % a.Hq, b = hb / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int chunk = qt / nqt_c;
  const int64_t qpos0 = chunk ? a.q_off2 : a.q_off;
  const int rank_e = chunk ? a.rank2 : a.rank;
  const int qrow0 = (qt - chunk * nqt_c) * BM;      // the workgroup's first row within the chunk
  const int qrow = qrow0 + lrow;
  const int my_q = chunk * nqc + qrow;
  const bool q_ok = qrow < nqc;

  float q[DL], o[DL];
  {
    const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)my_q * a.q_ss + (int64_t)h * a.q_sh + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (q_ok) x = *(const f32x4*)(qp + c);
      q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
    }
  }
  // running max m2 (log2 units of the scaled logits) and sum l, the same in
  // both lanes of a row
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) o[c] = 0.f;
  if (a.state_in && q_ok) {
    const float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4) {
      f32x4 x = *(const f32x4*)(op + c);
      o[c] = x[0]; o[c + 1] = x[1]; o[c + 2] = x[2]; o[c + 3] = x[3];
    }
    m2 = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss] * kLog2e;
    lsum = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss];
  }

  const int64_t q0_wg = qpos0 + qrow0;
  const int nq_wg = min(BM, nqc - qrow0);
  const int64_t qpos = qpos0 + qrow;
  const int nsteps = a.ring ? a.P : 1;
  for (int s = 0; s < nsteps; ++s) {
    const int64_t jb = a.ring ? ra_plan_ring_block(a.P, rank_e, s) : 0;
    const int64_t kv_off = a.ring ? jb * a.nkv : a.kv_off;
    const int64_t row0 = a.ring ? jb * a.nkv : 0;
    const int64_t nkeys = a.kv_end - kv_off < 0 ? 0 : (a.kv_end - kv_off < a.nkv ? a.kv_end - kv_off : a.nkv);
    const int nt = (int)ra_plan_key_tiles(q0_wg, nq_wg, kv_off, nkeys, a.causal, BN);
    for (int u = 0; u < nt; ++u) {
      const int64_t left = nkeys - (int64_t)u * BN;
      const int nvalid = left < BN ? (int)left : BN;
      const float* kb = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh + (row0 + (int64_t)u * BN) * a.k_ss;
      const float* vb = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh + (row0 + (int64_t)u * BN) * a.v_ss;
      __syncthreads();
      for (int id = tid; id < BN * D / 4; id += NT) {
        const int r = id / (D / 4), c4 = id % (D / 4);
        f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
        if (r < nvalid) {
          kx = *(const f32x4*)(kb + (int64_t)r * a.k_ss + 4 * c4);
          vx = *(const f32x4*)(vb + (int64_t)r * a.v_ss + 4 * c4);
        }
        *(f32x4*)(Ks + r * D + 4 * c4) = kx;
        *(f32x4*)(Vs + r * D + 4 * c4) = vx;
      }
      __syncthreads();
      const int64_t k0 = kv_off + (int64_t)u * BN;
      // visible keys of this row in the tile: a prefix of lim
      const int lim = (int)ra_plan_visible_prefix(qpos, k0, nvalid, a.causal);
      for (int j0 = 0; j0 < BN; j0 += CH) {
        if (j0 >= lim) break;  // the rest of the tile is masked for this row (uniform per wave when it matters)
        float sc[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const float* kr = Ks + (j0 + j) * D + c0;
          float dot = 0.f;
#pragma unroll
          for (int c = 0; c < DL; c += 4) {
            const f32x4 kx = *(const f32x4*)(kr + c);
            dot = fmaf(q[c], kx[0], dot);
            dot = fmaf(q[c + 1], kx[1], dot);
            dot = fmaf(q[c + 2], kx[2], dot);
            dot = fmaf(q[c + 3], kx[3], dot);
          }
          if constexpr (LPR == 2) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
            dot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          }
          sc[j] = j0 + j < lim ? dot * a.c : -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < CH; ++j) mx = fmaxf(mx, sc[j]);
        const float m_new = fmaxf(m2, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        if (m_new > m2) {  // rescale only when the max grows (alpha = 0 when m2 was -inf)
          const float alpha = exp2f(m2 - m_use);
          lsum *= alpha;
#pragma unroll
          for (int c = 0; c < DL; ++c) o[c] *= alpha;
          m2 = m_new;
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const float p = exp2f(sc[j] - m_use);
          lsum += p;
          const float* vr = Vs + (j0 + j) * D + c0;
#pragma unroll
          for (int c = 0; c < DL; c += 4) {
            const f32x4 vx = *(const f32x4*)(vr + c);
            o[c] = fmaf(p, vx[0], o[c]);
            o[c + 1] = fmaf(p, vx[1], o[c + 1]);
            o[c + 2] = fmaf(p, vx[2], o[c + 2]);
            o[c + 3] = fmaf(p, vx[3], o[c + 3]);
          }
        }
      }
    }
  }

  if (!q_ok) return;
  if (a.out_state) {
    float* op = a.oacc + (int64_t)b * a.oa_sb + (int64_t)my_q * a.oa_ss + (int64_t)h * a.oa_sh + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4) *(f32x4*)(op + c) = f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]};
    if (half == 0) {
      a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + (int64_t)my_q * a.m_ss] = m2 * kLn2;
      a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + (int64_t)my_q * a.l_ss] = lsum;
    }
  } else {
    const float inv = 1.f / lsum;
    const int64_t base = (int64_t)b * a.o_sb + (int64_t)my_q * a.o_ss + (int64_t)h * a.o_sh + c0;
    if (a.o_bf16) {
      __bf16* op = (__bf16*)a.o + base;
#pragma unroll
      for (int c = 0; c < DL; c += 4)
        *(bf16x4*)(op + c) = bf16x4{(__bf16)(o[c] * inv), (__bf16)(o[c + 1] * inv),
                                    (__bf16)(o[c + 2] * inv), (__bf16)(o[c + 3] * inv)};
    } else {
      float* op = (float*)a.o + base;
#pragma unroll
      for (int c = 0; c < DL; c += 4)
        *(f32x4*)(op + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
    }
    if (half == 0 && a.lse)
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)my_q * a.lse_ss] = m2 * kLn2 + logf(lsum);
  }
}

}  // namespace

hipError_t ra_launch_attn_bf16(const RaAttnArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)(ra_query_tiles(a, RA_BF16_BM) * a.Hq * a.B)), block(RA_BF16_THREADS);
  if (d == 128) hipLaunchKernelGGL(attn_bf16_w64_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_bf16_w64_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_attn_f32(const RaAttnArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)(ra_query_tiles(a, RA_F32_BM) * a.Hq * a.B)), block(64 * (d / 64));
  if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}
