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
// bf16 path (attn_bf16_w64_kernel).  One workgroup = 4 waves = 256 query
// rows of one head, one wave per SIMD; each wave owns 64 query rows as two
// 32-row blocks.  Keys come in tiles of 64, processed as two 32-key units:
//   S^T (keys x queries) = K Q^T   v_mfma_f32_32x32x16_bf16; K from LDS is the
//                                  A operand, the Q fragments stay in AGPRs
//                                  for the whole kernel as the B operand
//   online softmax                 the accumulator layout puts one query per
//                                  lane (lane & 31) and 16 of the unit's 32
//                                  keys in that lane's registers (the other
//                                  16 sit in lane ^ 32)
//   O^T (channels x queries) += V^T P^T   P^T goes from registers straight
//                                  into the B operand (bf16, round to nearest
//                                  even); the A operand V^T comes from
//                                  row-major V in LDS through the transposing
//                                  ds_read_b64_tr_b16; the accumulators sit
//                                  in AGPRs
// Every K and V^T fragment a wave reads from LDS feeds the MFMAs of both of
// its row blocks.  Per wave, a software pipeline with one step per unit u:
// the MFMAs of S(u+1) and of O += V(u-1) P(u-1) interleaved with the vector
// work of the softmax of S(u), which depends on neither.
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
// The fp32 path is in ra_f32.hip.
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

// attn_bf16_w64_kernel: the register file holds the output accumulators
// of both row blocks (2 x D/32 x 16 fp32) in AGPRs, pinned there by the P V
// products being inline-asm MFMAs.  A SIMD's matrix core is fed by one
// instruction stream, so each pipeline step alternates single MFMAs with
// short runs of the softmax's vector work (16 slots of two MFMAs per 32-key
// unit).

// The MFMAs of attn_bf16_w64_kernel, inline asm so that the operands sit in
// the register file the kernel needs them in (the builtins leave that to the
// compiler, which then runs out of VGPRs and copies between the files).
// The wait states around them (gfx950, as the compiler spaces its own
// MFMAs: 2 after a vector write of an operand, none between dependent
// products, 12 before a vector read of a result):
//   - after a vector write of an operand: none is needed where the products
//     sit (P is written a step before its product, the V^T and K fragments
//     come from LDS reads, the Q fragments are written once before the first
//     product, which has its own s_nop, and a redo's rescale of O comes
//     eight slots before the next P V product); the compiler also spaces an
//     asm statement from vector writes before it.  A leading s_nop 1 on the
//     P V product cost 3 % of the kernel's cycles;
//   - before a vector read of a result: the kernel's drains (16 wait
//     states), and otherwise whole pipeline slots between the write and the
//     read.
// Both are checked in the kernel's assembly by the tests.
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
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(A), "v"(B));
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
  // Rows past the block read the tensor's first row: finite, and never
  // stored.  The loads all go out here, with no wait between them; the
  // fragments are pinned to AGPRs once the prologue's tile loads are out too.
  bf16x8 qf[RB][KC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)(q_ok[rb] ? my_q[rb] : 0) * a.q_ss +
                       (int64_t)h * a.q_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[rb][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 16 * c));
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
    if (a.state_in) {  // rows past the block read the first row's state: never stored
      const int64_t row = q_ok[rb] ? my_q[rb] : 0;
      const float* op = a.oacc + (int64_t)b * a.oa_sb + row * a.oa_ss + (int64_t)h * a.oa_sh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 x = *(const f32x4*)(op + 32 * db + 8 * j + 4 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][db][4 * j + i] = x[i];
        }
      const float mv = a.m[(int64_t)b * a.m_sb + (int64_t)h * a.m_sh + row * a.m_ss];
      const float lv = a.l[(int64_t)b * a.l_sb + (int64_t)h * a.l_sh + row * a.l_ss];
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
  auto step_keys = [&](int s) -> int64_t {
    const int64_t n = a.kv_end - step_kv_off(s);
    return n < 0 ? 0 : (n < a.nkv ? n : a.nkv);
  };
  auto step_tiles = [&](int s) -> int {
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, step_kv_off(s), step_keys(s), a.causal, BN);
  };

  // Direct loads.  All four waves load a share (NL KiB) of each K and V
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
    // Cursor over the tiles: loop step cs, tile cu of its cnt tiles, the
    // tile's key position relative to the wave's first query (saturated at
    // +-2^30: a tile that far before the queries is fully visible, one that
    // far after them is never walked under causal masking, and the position
    // is not used without it; a block holds at most 2^29 keys, so the
    // position stays on its side of zero), keys left in the block from it
    // on, K and V addresses of its first row.
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

    // Mask of row block rb's unit (the wave's rows 32 rb ..), whose S^T is in
    // sacc[x], at key position k0 with nvalid valid keys (a rare branch
    // before the step's region): keys kvi < lim of the unit are visible to
    // this lane's query: lim = valid keys, cut at the query's own position
    // under causal masking (0 when the whole unit lies after it: p = 0).  The
    // key index of register r is 8 (r / 4) + (r % 4) + 4 lg.
    auto sm_mask = [&](int x, int rb, int64_t k0, int nvalid) __attribute__((always_inline)) {
      const int64_t q0r = q0w + 32 * rb;
      if (__builtin_expect(ra_plan_tile_masked<int64_t>(k0 - q0r, nvalid, 32, a.causal), 0)) {
        const int lim = (int)ra_plan_visible_prefix(q0r + lr, k0, nvalid, a.causal) - 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[x][rb][r] = (8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : sacc[x][rb][r];
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
    //
    // Softmax sub-step j of a step (row block j % 2, keys 2k, 2k+1 of the
    // lane's 16 with k = j / 2), software-pipelined over the slots: the
    // exponent arguments of sub-step j are formed in the slot before, so a
    // slot runs the bf16 P of sub-step j - 1 and the two exponentials (sm_a)
    // under one MFMA and the sums and the next sub-step's arguments (sm_b)
    // under the other.  The conversion goes first: the compiler keeps a wait
    // state between an MFMA and an exponential right behind it, which the
    // conversion fills (the last sub-step's is converted after the slots).
    float sm_ps[RB][4], sm_tot[RB] = {0.f, 0.f}, sm_p[RB][2], sm_arg[2];
    auto sm_args = [&](auto X, auto J) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, j = decltype(J)::value, rb = j % 2, k = j / 2;
      const f32x16& s = sacc[x][rb];
      sm_arg[0] = fmaf(s[2 * k], a.c, -m2[rb]);
      sm_arg[1] = fmaf(s[2 * k + 1], a.c, -m2[rb]);
      asm volatile("" : "+v"(sm_arg[0]), "+v"(sm_arg[1]));
    };
    // bf16 P of sub-step 2k + rb (its two exponentials, still in sm_p[rb])
    auto sm_cvt = [&](auto X, auto R, auto K) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, rb = decltype(R)::value, k = decltype(K)::value;
      pf[x][rb][k >> 2][2 * (k & 3)] = (__bf16)sm_p[rb][0];
      pf[x][rb][k >> 2][2 * (k & 3) + 1] = (__bf16)sm_p[rb][1];
      asm volatile("" : "+v"(pf[x][rb][k >> 2]));
    };
    auto sm_a = [&](auto X, auto R, auto K) __attribute__((always_inline)) {
      constexpr int rb = decltype(R)::value, j = 2 * decltype(K)::value + rb;
      if constexpr (j > 0) sm_cvt(X, std::integral_constant<int, (j - 1) % 2>{}, std::integral_constant<int, (j - 1) / 2>{});
      __builtin_amdgcn_sched_barrier(0);
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
      asm volatile("" : "+v"(sm_ps[rb][k & 3]));
      if constexpr (k == 7) {
        sm_tot[rb] = (sm_ps[rb][0] + sm_ps[rb][1]) + (sm_ps[rb][2] + sm_ps[rb][3]);
        asm volatile("" : "+v"(sm_tot[rb]));
      }
    };
    // After the step: redo a row block's unit if any lane asks for it (the
    // row sum is added after, in sm_fix).  The redo moves m2 to the exact row
    // max, rescales o and l by alpha = exp2(m2_old - m2_new) (0 when m2 was
    // -inf) and recomputes p (0 for rows with no visible key yet).
    auto sm_redo = [&](auto X, auto R) __attribute__((always_inline)) {
      constexpr int x = decltype(X)::value, rb = decltype(R)::value;
      if (__builtin_amdgcn_ballot_w64(!(sm_tot[rb] <= kRedoSum)) != 0) {
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
    };
    // One test for both row blocks on the common path (a lane's sums in
    // range); the redo of each row block behind it.
    auto sm_fix = [&](auto X) __attribute__((always_inline)) {
      const bool bad = !(sm_tot[0] <= kRedoSum) || !(sm_tot[1] <= kRedoSum);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) {
        sm_redo(X, std::integral_constant<int, 0>{});
        sm_redo(X, std::integral_constant<int, 1>{});
      }
      lsum[0] += sm_tot[0];
      lsum[1] += sm_tot[1];
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
        sm_cvt(X, std::integral_constant<int, 1>{}, std::integral_constant<int, 7>{});
        sm_fix(X);
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
    const integral_constant<int, 0> X0, H0;
    const integral_constant<int, 1> X1, H1;

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
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("" : "+a"(qf[rb][c]));  // from here on the fragments live in AGPRs
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

}  // namespace

hipError_t ra_launch_attn_bf16(const RaAttnArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)(ra_query_tiles(a, RA_BF16_BM) * a.Hq * a.B)), block(RA_BF16_THREADS);
  if (d == 128) hipLaunchKernelGGL(attn_bf16_w64_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_bf16_w64_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}
