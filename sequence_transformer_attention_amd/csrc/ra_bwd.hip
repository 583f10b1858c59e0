// ra_bwd.hip -- gfx950 kernels of the backward of one rank's share.
//
// What is computed (glossary page "sequence parallelism transformers",
// section "Implementation Considerations", item "Gradient Synchronization":
// the backward pass needs the same communication as the forward pass): the
// gradients of the share's outputs O with respect to its local queries and,
// for every key of the sequence, this rank's contribution to dK and dV (the
// part the ring would carry back to the key's owner).  With the forward's
// P_ij = exp(s_ij - LSE_i), s_ij = scale <q_i, k_j>, and dO the gradient
// arriving at O:
//   D_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i
// P is recomputed from the saved LSE (no softmax state is kept).
//
// Kernels (bf16 inputs, fp32 accumulation, v_mfma_f32_32x32x16_bf16):
//   bwd_prep_kernel   D_i, one thread per row.
//   bwd_dq_kernel     4 waves x 32 query rows (Q and dO fragments stay in
//                     registers as B operands); per 32-key unit of a
//                     64-key K/V tile staged in LDS:
//                       S^T = K Q^T, then dP^T = V dO^T (A operands from
//                       LDS), dS^T = P^T (dP^T - D) in fp32, then
//                       dQ^T += K^T dS^T with K^T from the transposing
//                       ds_read_b64_tr_b16 and dS^T from registers.  Each
//                       product phase issues the LDS reads of the next into
//                       the registers its own MFMAs free (V rows during S^T,
//                       K^T during dP^T, the next unit's K rows during dQ^T).
//                     256 VGPRs: two workgroups (two waves per SIMD) per CU.
//   bwd_dkdv_kernel   4 waves x 32 keys (K and V fragments and the dK, dV
//                     accumulators in AGPRs for the whole walk: inline-asm
//                     MFMAs); per 32-query unit of a 128-row Q/dO tile
//                     staged in LDS, for every query head of the kv head:
//                       S = Q K^T, then dP = dO V^T (A operands from LDS)
//                       with P formed between its MFMAs, dV^T += dO^T P
//                       (dO^T from transposing reads) with dS formed
//                       between its MFMAs, dK^T += Q^T dS, each phase
//                       issuing the LDS reads of the next.  One wave per
//                       SIMD issues both streams: scheduling barriers keep
//                       the vector work between the MFMAs, where it issues
//                       while the matrix core runs.
// Both attention kernels use the forward's LDS layout (rows of 2d bytes,
// 16-byte slots XOR-swizzled), two LDS stages with the next tile's loads in
// flight, and inline-asm LDS reads whose waits carry their registers.
#include "ra_bwd.h"
#include "ra_plan.h"

#include <type_traits>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kLog2e = 1.4426950408889634f;

// Physical 16-byte slot of logical slot p in LDS row r (the forward's swizzle:
// conflict-free 128-bit reads of 16 rows at one slot and transposing reads).
template <int SLOTS>
__device__ __forceinline__ int swz(int r, int p) {
  return p ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (SLOTS - 1));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Per-lane LDS addresses inside a 64-row tile (rows of 2D bytes):
//   rd[c]:        128-bit read of row lr, logical slot 2c + lg (A operand of
//                 a 32x32x16 MFMA: row lr, elements 16c + 8lg .. +7);
//   tr[half][db]: transposing read, as the forward's V^T reads (A operand
//                 of channel block db over 16 rows; + 2D * 16 hh per group).
template <int D>
struct TileAddr {
  static constexpr int SLOTS = D / 8, KC = D / 16, DB = D / 32;
  unsigned rd[KC], tr[2][DB];
  __device__ __forceinline__ void init(unsigned base, int lane) {
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int c = 0; c < KC; ++c) rd[c] = base + lr * 2 * D + 16 * swz<SLOTS>(lr, 2 * c + lg);
    const int vj = lane & 15, ve = vj >> 2, vc = vj & 3, vgrp = lane >> 4;
    const int vx = 2 * (vgrp & 1) + (vc >> 1);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r = 4 * lg + ve + 8 * half;
        tr[half][db] = base + r * 2 * D + 16 * swz<SLOTS>(r, 4 * db + vx) + 8 * (vc & 1);
      }
  }
};

// LDS reads with an immediate byte offset.
template <unsigned OFF, typename T>
__device__ __forceinline__ void ds_rd128(T& r, unsigned addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <unsigned OFF>
__device__ __forceinline__ void ds_rdtr(u32x2& r, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}

// acc[i] += A_i * B (v_mfma_f32_32x32x16_bf16, i = 0..3) with the
// accumulators pinned to AGPRs.  An MFMA needs 2 wait states after a vector
// write of its operands (gfx950, as the compiler spaces its own MFMAs); the
// compiler spaces an asm statement from the vector writes before it, which
// the tests check in the assembly.  Only other MFMAs of this form touch the
// accumulators until mfma_acc_drain.
__device__ __forceinline__ void mfma_acc4(f32x16& c0, f32x16& c1, f32x16& c2, f32x16& c3, const u32x4& a0,
                                          const u32x4& a1, const u32x4& a2, const u32x4& a3, const bf16x8& b) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %5, %8, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %6, %8, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %7, %8, %3"
      : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b));
}
// acc += A * B, one v_mfma_f32_32x32x16_bf16 with the accumulator pinned to
// AGPRs (as mfma_acc4, for interleaving with vector work).
__device__ __forceinline__ void mfma_acc1(f32x16& c, const u32x4& A, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(A), "v"(b));
}
// Zero an accumulator with an MFMA (zero operands, inline-constant C), so
// that it is born in AGPRs.
__device__ __forceinline__ void mfma_acc_zero(f32x16& c) {
  const bf16x8 z = bf16x8{};
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(c) : "v"(z));
}
// Wait until the MFMAs writing the accumulators are done before anything
// else reads them (the compiler gives a vector read of an 8-pass MFMA's
// result 12 wait states; 16 are given).
__device__ __forceinline__ void mfma_acc_drain(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(c));
}

// Load a 64-row tile (rows row0 .. row0 + nvalid - 1 of a [*, D] bf16 matrix
// with row stride `stride` elements, at most 2^24; nvalid <= 64) into LDS at
// dst, swizzled.  All NW waves take a share of 1 KiB chunks.  The buffer
// range ends at row nvalid - 1 (is empty for nvalid <= 0), so rows past it
// are out of range: nothing is fetched for them and their LDS bytes are
// written as zeros.
template <int D, int NW>
__device__ __forceinline__ void load_tile(const __bf16* row0, int64_t stride, int nvalid, char* dst, int wave,
                                          int lane) {
  constexpr int SLOTS = D / 8, TILE = 64 * D * 2, NL = TILE / 1024 / NW;
  const int nrec = nvalid > 0 ? (nvalid - 1) * (int)stride * 2 + 2 * D : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)row0, (short)0, nrec, 0x00020000);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int ls = (wave * NL + i) * 64 + lane;
    const int r = ls / SLOTS;
    const unsigned off = (unsigned)r * (unsigned)stride * 2u + 16u * (unsigned)swz<SLOTS>(r, ls % SLOTS);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + (wave * NL + i) * 1024), 16, off, 0, 0, 0);
  }
}

// D_i = <dO_i, O_i> for every local row.
__global__ void __launch_bounds__(256) bwd_prep_kernel(RaBwdArgs a, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.B * a.Hq * a.nq) return;
  const int i = (int)(idx % a.nq);
  const int64_t t = idx / a.nq;
  const int h = (int)(t % a.Hq), b = (int)(t / a.Hq);
  const __bf16* op = (const __bf16*)a.o + (int64_t)b * a.o_sb + (int64_t)i * a.o_ss + (int64_t)h * a.o_sh;
  const __bf16* dp = (const __bf16*)a.dout + (int64_t)b * a.do_sb + (int64_t)i * a.do_ss + (int64_t)h * a.do_sh;
  float s = 0.f;
  for (int c = 0; c < d; c += 8) {
    const bf16x8 x = *(const bf16x8*)(op + c), y = *(const bf16x8*)(dp + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
  }
  a.delta[(int64_t)b * a.de_sb + (int64_t)h * a.de_sh + (int64_t)i * a.de_ss] = s;
}

template <int D>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(RaBwdArgs a) {
  constexpr int NW = 4, BM = NW * 32, BN = RA_BWD_BN, KC = D / 16, DB = D / 32, TILE = BN * D * 2;
  static_assert(BM == RA_BWD_BM, "query rows per workgroup");
  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // two stages of (K tile, V tile)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  // query chunks (two under the load-balanced split), each with its own
  // positions and ring order over Pe blocks of nbe keys
  const int nqc = a.nsplit == 2 ? (int)a.qc : a.nq;
  const int nqt_c = (nqc + BM - 1) / BM, nqt = a.nsplit * nqt_c;
  const int logical = ra_plan_xcd_remap(blockIdx.x, gridDim.x, nqt);
  int qt = logical % nqt;
  const int hb = logical / nqt;
  if (a.causal) qt = nqt - 1 - qt;  // later query tiles see more keys: start them first
  const int chunk = qt / nqt_c;
  const int64_t qpos0 = chunk ? a.q_off2 : a.q_off;  // position of the chunk's first row
  const int rank_e = chunk ? a.rank2 : a.rank, Pe = a.nsplit * a.P;
  const int64_t nbe = a.nsplit == 2 ? a.qc : a.nb;
  const int h = hb % a.Hq, b = hb / a.Hq, hk = h / (a.Hq / a.Hkv);
  const int qrow_wg = (qt - chunk * nqt_c) * BM, qrow_w = qrow_wg + wave * 32;  // rows within the chunk
  const int my_q = chunk * nqc + qrow_w + lr;                                  // local row
  const bool q_ok = qrow_w + lr < nqc;

  bf16x8 qf[KC], dof[KC];  // lane: row my_q, elements 16c + 8lg .. +7
  {
    const int row = q_ok ? my_q : 0;
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)row * a.q_ss + (int64_t)h * a.q_sh + 8 * lg;
    const __bf16* dp =
        (const __bf16*)a.dout + (int64_t)b * a.do_sb + (int64_t)row * a.do_ss + (int64_t)h * a.do_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      qf[c] = q_ok ? *(const bf16x8*)(qp + 16 * c) : bf16x8{};
      dof[c] = q_ok ? *(const bf16x8*)(dp + 16 * c) : bf16x8{};
    }
  }
  // rows past nq: LSE = +inf gives P = 0
  const float lse2 = q_ok ? a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)my_q * a.lse_ss] * kLog2e
                          : INFINITY;
  const float dlt = q_ok ? a.delta[(int64_t)b * a.de_sb + (int64_t)h * a.de_sh + (int64_t)my_q * a.de_ss] : 0.f;

  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};
  TileAddr<D> ta;
  ta.init((unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)&smem[0][0][0]), lane);

  const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh;
  const int64_t q0_wg = qpos0 + qrow_wg, q0w = qpos0 + qrow_w;
  const int nq_wg = min(BM, nqc - qrow_wg);
  // Key block of loop step s: ring order with the rank's own block (ring
  // step 0) last, so that all query tiles of a head walk the other blocks in
  // lockstep and share the K/V stream in L2 (the own block's causal tile
  // count differs per query tile).
  auto blk = [&](int s) -> int64_t { return ra_plan_ring_block(Pe, rank_e, (s + 1) % Pe); };
  // keys of block b0 * nbe .. before the key end
  auto blk_keys = [&](int64_t k0) -> int64_t {
    const int64_t n = a.kv_end - k0;
    return n < 0 ? 0 : (n < nbe ? n : nbe);
  };
  auto tiles = [&](int s) -> int {
    const int64_t k0 = blk(s) * nbe;
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, k0, blk_keys(k0), a.causal, BN);
  };
  // The workgroup's key tiles in that order; the loads of the next tile are
  // in flight while the current one is computed (two LDS stages).
  struct Cur {
    int s, u, nt;
    int64_t k0;
  };
  auto cur_fix = [&](Cur& c) {  // move to the first tile of the first non-empty step from c.s on
    while (c.s < Pe && (c.nt = tiles(c.s)) == 0) ++c.s;
    c.u = 0;
    c.k0 = c.s < Pe ? blk(c.s) * nbe : 0;
  };
  auto cur_next = [&](Cur& c) {
    if (++c.u < c.nt) return;
    ++c.s;
    cur_fix(c);
  };
  int total = 0;
  for (int s = 0; s < Pe; ++s) total += tiles(s);
  Cur cc{0, 0, 0, 0}, cl{0, 0, 0, 0};  // compute cursor, load cursor
  cur_fix(cc);
  cur_fix(cl);
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int64_t k0 = cl.k0 + (int64_t)cl.u * BN, left = blk_keys(cl.k0) - (int64_t)cl.u * BN;
    const int nvalid = left < BN ? (int)left : BN;
    load_tile<D, NW>(kb + k0 * a.k_ss, a.k_ss, nvalid, &smem[st][0][0], wave, lane);
    load_tile<D, NW>(vb + k0 * a.v_ss, a.v_ss, nvalid, &smem[st][1][0], wave, lane);
    cur_next(cl);
  };
  // K rows of the unit (A operand of S^T), read a unit ahead within a tile
  bf16x8 fk[KC];
  auto read_k = [&](auto KO) __attribute__((always_inline)) {
    static_for<0, KC>([&](auto C) { ds_rd128<decltype(KO)::value>(fk[decltype(C)::value], ta.rd[decltype(C)::value]); });
  };
  auto tile = [&](int it, auto ST) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    const int64_t k0 = cc.k0 + (int64_t)cc.u * BN, left = blk_keys(cc.k0) - (int64_t)cc.u * BN;
    const int nvalid = left < BN ? (int)left : BN;
    cur_next(cc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // publishes stage st; every wave is done with stage st ^ 1
    read_k(std::integral_constant<unsigned, (unsigned)st * 2 * TILE>{});  // the tile's only exposed reads
    if (it + 1 < total) issue(st ^ 1);
    static_for<0, 2>([&](auto HF) {
      constexpr int hf = decltype(HF)::value;
      constexpr unsigned ko = (unsigned)st * 2 * TILE + (unsigned)hf * 64 * D;  // K unit; V unit at + TILE
      // Each phase issues the LDS reads of the next, into the registers its
      // products free: the V rows during the S^T products, K^T during the
      // dP^T products, the next unit's K rows during the dQ products.
      if constexpr (KC == 8)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fk[0]), "+v"(fk[1]), "+v"(fk[2]), "+v"(fk[3]), "+v"(fk[4]),
                     "+v"(fk[5]), "+v"(fk[6]), "+v"(fk[7]));
      else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fk[0]), "+v"(fk[1]), "+v"(fk[2]), "+v"(fk[3]));
      // S^T = K Q^T (keys x queries)
      f32x16 sacc = f32x16{}, dpa = f32x16{};
      bf16x8 fv[KC];
      static_for<0, KC>([&](auto C) {
        constexpr int c = decltype(C)::value;
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[c], qf[c], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        ds_rd128<ko + TILE>(fv[c], ta.rd[c]);
        __builtin_amdgcn_sched_barrier(0);
      });
      // dP^T = V dO^T
      u32x2 tlo[2][DB], thi[2][DB];
      static_for<0, KC>([&](auto C) {
        constexpr int c = decltype(C)::value, hh = c / DB, d_ = c % DB;
        // fv[c] done: the reads after it are fv[c + 1 ..] and c pairs of K^T
        constexpr int n = KC - 1 + c < 14 ? KC - 1 + c : 14;
        asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fv[c]) : "n"(n));
        dpa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[c], dof[c], dpa, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        constexpr unsigned off = ko + (unsigned)hh * 32 * D;
        ds_rdtr<off>(tlo[hh][d_], ta.tr[0][d_]);
        ds_rdtr<off>(thi[hh][d_], ta.tr[1][d_]);
        __builtin_amdgcn_sched_barrier(0);
      });
      // key index of register r: 8 (r / 4) + (r % 4) + 4 lg; keys below lim are visible
      const int nv = ra_plan_half_valid(nvalid, hf, 32);
      bf16x8 dsf[2];
      // all 32 keys of the unit exist and precede the wave's first query: no test
      if (!ra_plan_tile_masked<int64_t>(k0 + 32 * hf - q0w, nv, 32, a.causal)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[r] * a.c - lse2);
          dsf[r >> 3][r & 7] = (__bf16)(p * (dpa[r] - dlt));
        }
      } else {
        const int lim = (int)ra_plan_visible_prefix(q0w + lr, k0 + 32 * hf, nv, a.causal);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + (r & 3) + 4 * lg;
          float t = __builtin_amdgcn_exp2f(sacc[r] * a.c - lse2);
          asm volatile("" : "+v"(t));  // computed for every lane: no branch
          const float p = kk < lim ? t : 0.f;
          dsf[r >> 3][r & 7] = (__bf16)(p * (dpa[r] - dlt));
        }
      }
      // dQ^T += K^T dS^T
      static_for<0, 2 * DB>([&](auto X) {
        constexpr int x = decltype(X)::value, hh = x / DB, d_ = x % DB;
        // K^T pair x done: the reads after it are the later pairs and the x
        // next K rows issued so far
        constexpr int pend = 2 * (2 * DB - 1 - x) + (hf == 0 ? x : 0);
        constexpr int n = pend < 14 ? pend : 14;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(tlo[hh][d_]), "+v"(thi[hh][d_]) : "n"(n));
        const u32x4 w = {tlo[hh][d_][0], tlo[hh][d_][1], thi[hh][d_][0], thi[hh][d_][1]};
        dqa[d_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), dsf[hh], dqa[d_], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (hf == 0 && x < KC) ds_rd128<ko + 64 * D>(fk[x], ta.rd[x]);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };
  if (total > 0) issue(0);
  for (int it = 0; it < total; it += 2) {
    tile(it, std::integral_constant<int, 0>{});
    if (it + 1 < total) tile(it + 1, std::integral_constant<int, 1>{});
  }
  if (!q_ok) return;
  float* dp = a.dq + (int64_t)b * a.dq_sb + (int64_t)my_q * a.dq_ss + (int64_t)h * a.dq_sh;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = {dqa[db][4 * j] * a.scale, dqa[db][4 * j + 1] * a.scale, dqa[db][4 * j + 2] * a.scale,
                       dqa[db][4 * j + 3] * a.scale};
      *(f32x4*)(dp + 32 * db + 8 * j + 4 * lg) = x;
    }
}

// S (queries x keys) = Q K^T and dP = dO V^T of the dK/dV kernel: A (Q or dO
// rows) in VGPRs, B (the lane's key: K or V) in AGPRs, the accumulator in
// VGPRs.  Inline asm (the compiler would keep K and V in VGPRs): before a
// vector read of the result the caller waits with qk_drain.
__device__ __forceinline__ void mfma_qk_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_qk_next(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// 12 wait states between the last MFMA writing c and a vector read of c,
// what gfx950 needs after an 8-pass MFMA (the callers place an independent
// product and its reads before it as well).
__device__ __forceinline__ void qk_drain(f32x16& c) { asm volatile("s_nop 7\n\ts_nop 3" : "+v"(c)); }

// dK and dV of one kv head for 128 keys per workgroup, 32 per wave (lane =
// key lr, both lane halves): K and V of the lane's key stay in AGPRs, the
// dK and dV accumulators too.  The query rows that see the keys are walked
// in tiles of QT = 128 rows (four 32-row units), Q and dO tiles staged in
// LDS in two stages with the next tile's loads in flight.  Per unit:
//   S = Q K^T, dP = dO V^T (8 + 8 MFMAs), P = exp2(S c - LSE log2 e)
//   under the causal mask, dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS
// with dO^T and Q^T from transposing LDS reads.  The LDS reads are issued
// a phase ahead of their products: a unit's dO rows during its S products,
// its dO^T during dP, its Q^T and the next unit's Q rows during dV, the
// next unit's row statistics during this unit's dK products (within a
// tile), so only the first unit of a tile waits for its Q rows.  The next tile's direct loads
// go out once the tile's first product runs (Q rows and statistics first).
template <int D>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(RaBwdArgs a) {
  constexpr int NW = 4, BK = NW * 32, QT = 128, NU = QT / 32, KC = D / 16, DB = D / 32;
  constexpr int TILE = QT * D * 2;           // one Q or dO tile
  constexpr unsigned DO_REGION = 2 * TILE;   // dO tiles follow both Q stages
  static_assert(2 * TILE <= 65536, "LDS offsets within a region fit the 16-bit immediate");
  // [Q stage 0 | Q stage 1 | dO stage 0 | dO stage 1]; row statistics
  // (LSE log2(e), D) of both stages
  __shared__ __attribute__((aligned(1024))) char smem[4][TILE];
  __shared__ __attribute__((aligned(16))) float lsd[2][2][QT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int nkt = (int)((a.N + BK - 1) / BK);
  const int logical = ra_plan_xcd_remap(blockIdx.x, gridDim.x, nkt);
  const int kt = logical % nkt, hb = logical / nkt;
  const int g = hb % a.Hkv, b = hb / a.Hkv, G = a.Hq / a.Hkv;
  const int64_t my_k = (int64_t)kt * BK + wave * 32 + lr;
  const bool k_ok = my_k < a.N;
  // a key before the key end; the others (padding) are read as zeros, see
  // no query and get zero gradients
  const bool k_live = my_k < a.kv_end;

  // lane: key my_k, elements 16c + 8lg .. +7, in AGPRs once these loads and
  // the first tile's are out (one wait, not one per load).  A key past the
  // key end reads the first key: its P is masked to 0, so it reaches nothing.
  bf16x8 kf[KC], vf[KC];
  {
    const int64_t row = k_live ? my_k : 0;
    const __bf16* kp = (const __bf16*)a.k + (int64_t)b * a.k_sb + row * a.k_ss + (int64_t)g * a.k_sh + 8 * lg;
    const __bf16* vp = (const __bf16*)a.v + (int64_t)b * a.v_sb + row * a.v_ss + (int64_t)g * a.v_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      kf[c] = *(const bf16x8*)(kp + 16 * c);
      vf[c] = *(const bf16x8*)(vp + 16 * c);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    mfma_acc_zero(dka[db]);
    mfma_acc_zero(dva[db]);
  }
  TileAddr<D> ta;  // per-lane addresses in a 64-row tile (offsets: region, stage, unit)
  ta.init((unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)&smem[0][0]), lane);
  const unsigned lsd_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) float*)&lsd[0][0][0]);
  const unsigned lsd_lane = lsd_base + 16u * (unsigned)lg;  // + 4 floats per lane group

  // The walk: (query head of the kv head, 128-row tile) pairs over the local
  // rows that see any key of the workgroup (under causal masking those at
  // positions >= the first key's, per query chunk), as in the 64-row form.
  const int64_t kfirst = (int64_t)kt * BK;
  const int64_t wave_klast = kfirst + wave * 32 + 31;  // the wave's last key
  const int nqc = a.nsplit == 2 ? (int)a.qc : a.nq;
  const int ntq = (nqc + QT - 1) / QT;  // tiles per chunk
  auto first_tile = [&](int64_t qpos) -> int { return ra_plan_first_query_tile(kfirst, qpos, nqc, QT, a.causal); };
  const int t0a = first_tile(a.q_off), t0b = a.nsplit == 2 ? first_tile(a.q_off2) : ntq;
  const int na = ntq - t0a, nt = na + (ntq - t0b);
  const int total = kfirst < a.kv_end ? G * nt : 0;  // no key before the key end: nothing to do
  struct TileRef {
    int h, r0, nvalid;
    int64_t qp0;
  };
  struct WalkCur {
    int h, w;
  };
  auto tile_ref = [&](const WalkCur& c) -> TileRef {
    const int ch = c.w >= na ? 1 : 0;
    const int t = ch ? t0b + (c.w - na) : t0a + c.w;
    TileRef r;
    r.h = g * G + c.h;
    r.r0 = ch * nqc + t * QT;
    r.nvalid = min(QT, nqc - t * QT);
    r.qp0 = (ch ? a.q_off2 : a.q_off) + (int64_t)t * QT;
    return r;
  };
  auto walk_next = [&](WalkCur& c) {
    if (++c.w == nt) {
      c.w = 0;
      ++c.h;
    }
  };
  WalkCur cl{0, 0}, cc{0, 0};  // load cursor, compute cursor
  // threads 0..QT-1: LSE and D of row tid of the tile in flight as loaded,
  // and whether the row exists; they are scaled and selected only when the
  // tile's statistics go to LDS (after the wait for the tile's loads), so
  // that issuing the loads waits for nothing
  float lsv = 0.f, dlv = 0.f;
  bool lok = false;
  // The loads of tile nx into stage st in four parts: Q rows 0-63 with the
  // rows' statistics (threads 0 .. QT-1), Q rows 64-127, dO rows 0-63, dO
  // rows 64-127.
  TileRef nx{0, 0, 0, 0};
  auto issue_part = [&](int st, int part) __attribute__((always_inline)) {
    const int h = nx.h, r0 = nx.r0, nvalid = nx.nvalid;
    const int half = part & 1;
    if (part < 2) {
      const __bf16* qrow = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)r0 * a.q_ss;
      load_tile<D, NW>(qrow + (int64_t)(64 * half) * a.q_ss, a.q_ss, nvalid - 64 * half,
                       &smem[st][0] + half * (TILE / 2), wave, lane);
    } else {
      const __bf16* drow = (const __bf16*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh + (int64_t)r0 * a.do_ss;
      load_tile<D, NW>(drow + (int64_t)(64 * half) * a.do_ss, a.do_ss, nvalid - 64 * half,
                       &smem[2 + st][0] + half * (TILE / 2), wave, lane);
    }
    if (part == 0 && tid < QT) {
      lok = tid < nvalid;
      const int row = r0 + (lok ? tid : 0);  // a tile has at least one row
      lsv = a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)row * a.lse_ss];
      dlv = a.delta[(int64_t)b * a.de_sb + (int64_t)h * a.de_sh + (int64_t)row * a.de_ss];
    }
  };
  auto issue = [&](int st) __attribute__((always_inline)) {
    nx = tile_ref(cl);
    walk_next(cl);
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(st, part);
  };

  // LDS reads are asm with immediate offsets, issued ahead of their
  // products and waited for with counts: LDS reads complete in order, and
  // at most 14 are waited on as outstanding (the counter has 4 bits; the
  // compiler's own waits stop at 14 as well).
  bf16x8 fq[KC];  // Q rows of the unit (A operand of S), read one unit ahead
  f32x4 l4[4];    // LSE log2(e) of the lane's 16 query rows (4 runs of 4), read with them
  // Unit v's Q row fragment c and its LSE.  The Q rows go first: the S
  // products wait for them one at a time, the LSE only the dP phase reads.
  auto read_q = [&](auto ST, auto V, auto C) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value, v = decltype(V)::value, c = decltype(C)::value;
    ds_rd128<(unsigned)st * TILE + (unsigned)v * 64 * D>(fq[c], ta.rd[c]);
  };
  auto read_l4 = [&](auto ST, auto V) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value, v = decltype(V)::value;
    constexpr unsigned o4 = ((unsigned)st * 2 * QT + 32u * v) * 4u;
    static_for<0, 4>([&](auto J) { ds_rd128<o4 + 32u * decltype(J)::value>(l4[decltype(J)::value], lsd_lane); });
  };
  auto read_q_l4 = [&](auto ST, auto V) __attribute__((always_inline)) {
    static_for<0, KC>([&](auto C) { read_q(ST, V, C); });
    read_l4(ST, V);
  };

  // One tile: stage ST (compile time, so every LDS offset is an immediate).
  // Per 32-row unit, the products run S, dP, dV, dK, and each phase issues
  // the reads of the next: the dO rows during S, dO^T during dP, Q^T and
  // the next unit's Q rows during dV, the next unit's LSE during dK.
  auto tile = [&](int it, auto ST) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    const int64_t qp0 = tile_ref(cc).qp0;
    walk_next(cc);
    // this lane's key relative to the tile's first query position (bounded
    // above by the tile walk; saturated below)
    const int64_t rel64 = my_k - qp0;
    const int rel = rel64 < -(1 << 30) ? -(1 << 30) : (int)rel64;
    // units from vfull on need no causal test (every key of the wave is
    // live and precedes their queries)
    const int vfull = ra_plan_first_full_unit(wave_klast, a.kv_end, qp0, NU, a.causal);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < QT) {
      lsd[st][0][tid] = lok ? lsv * kLog2e : INFINITY;  // rows past the chunk: P = 0
      lsd[st][1][tid] = lok ? dlv : 0.f;
    }
    __syncthreads();  // publishes stage st; every wave is done with stage st ^ 1
    const bool more = it + 1 < total;
    if (more) {
      nx = tile_ref(cl);
      walk_next(cl);
    }
    read_q_l4(ST, std::integral_constant<int, 0>{});  // the tile's only exposed reads
    static_for<0, NU>([&](auto V) {
      constexpr int v = decltype(V)::value;
      constexpr unsigned qo = (unsigned)st * TILE + (unsigned)v * 64 * D;  // unit v; dO at + DO_REGION
      // S = Q K^T (query row of register r: 8 (r / 4) + 4 lg + (r % 4)),
      // with the dO rows read one per product, then D of the rows.  Each
      // product waits for its own Q fragment: the reads after fq[c] are the
      // later fragments, the unit's four LSE reads and the c dO rows read so
      // far.  Only the asm products read the Q and dO fragments, and
      // volatile asm keeps its order, so the waits take them as inputs: as
      // outputs the compiler counts a wait as a vector write and puts an
      // s_nop before the next product.
      f32x16 sacc;
      bf16x8 fd[KC];
      static_for<0, KC>([&](auto C) {
        constexpr int c = decltype(C)::value;
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(KC + 3), "v"(fq[c]));
        if constexpr (c == 0) {
          mfma_qk_first(sacc, fq[0], kf[0]);
          // the next tile's loads, once the tile's first product runs
          if constexpr (v == 0)
            if (more) {
#pragma unroll
              for (int part = 0; part < 4; ++part) issue_part(st ^ 1, part);
            }
        } else {
          mfma_qk_next(sacc, fq[c], kf[c]);
        }
        ds_rd128<qo>(fd[c], ta.rd[c] + DO_REGION);
      });
      f32x4 d4[4];
      static_for<0, 4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        ds_rd128<((unsigned)st * 2 * QT + QT + 32u * v + 8u * j) * 4u>(d4[j], lsd_lane);
      });
      // visible: under causal masking, the query at position qp0 + 32 v +
      // 4 lg + e (e = 8 (r / 4) + (r % 4)) is at or after this lane's key:
      // e >= lo.  Rows past their chunk need no test (their LSE is +inf:
      // P = 0, and D = 0), nor keys past the sequence (their P only reaches
      // their own dK, dV columns, which are not stored).
      const int lo = !k_live ? (1 << 30) : (a.causal ? rel - 32 * v - 4 * lg : -(1 << 30));
      // dP = dO V^T, one MFMA per slot; each slot also issues one pair of
      // dO^T reads and forms 16 / KC elements of P.  The first slot's
      // product does not read S: it goes out before S's drain and runs
      // through it.
      constexpr int PE = 16 / KC;
      f32x16 dpa;
      float pv[16];
      bf16x8 pf[2];
      u32x2 olo[2][DB], ohi[2][DB], qlo[2][DB], qhi[2][DB];
      static_for<0, KC>([&](auto C) {
        constexpr int c = decltype(C)::value, hh = c / DB, d_ = c % DB;
        // fd[c] done: the reads after it are fd[c + 1 ..], D and c pairs
        // (the LSE, read before the dO rows, is done with fd[0]: it feeds
        // compiled arithmetic and is an output there)
        constexpr int n = KC + 3 + c < 14 ? KC + 3 + c : 14;
        if constexpr (c == 0)
          asm volatile("s_waitcnt lgkmcnt(%4)"
                       : "+v"(l4[0]), "+v"(l4[1]), "+v"(l4[2]), "+v"(l4[3])
                       : "n"(n), "v"(fd[c]));
        else
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(n), "v"(fd[c]));
        if constexpr (c == 0) mfma_qk_first(dpa, fd[0], vf[0]);
        else mfma_qk_next(dpa, fd[c], vf[c]);
        ds_rdtr<qo + (unsigned)hh * 32 * D>(olo[hh][d_], ta.tr[0][d_] + DO_REGION);
        ds_rdtr<qo + (unsigned)hh * 32 * D>(ohi[hh][d_], ta.tr[1][d_] + DO_REGION);
        if constexpr (c == 0) qk_drain(sacc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < PE; ++q) {
          const int r = PE * c + q;
          pv[r] = __builtin_amdgcn_exp2f(sacc[r] * a.c - l4[r >> 2][r & 3]);
          pf[r >> 3][r & 7] = (__bf16)pv[r];
          // packed here, among the products (not sunk past the mask below)
          if ((r & 7) == 7) asm volatile("" : "+v"(pf[r >> 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // P above is formed without the mask (a term the mask drops may be
      // inf: the select below discards it).  The mask is applied only where
      // some element needs it: a query of the unit before a key of the wave,
      // or a key of the wave past the key end (the units on the diagonal, or
      // at the sequence's end).  Done for every unit, the test and select
      // cost about 7 % of the kernel's cycles; here the other units pass by
      // on one branch on a wave-uniform value.
      if (v < vfull) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 8 * (r >> 2) + (r & 3);
          pv[r] = e >= lo ? pv[r] : 0.f;
          pf[r >> 3][r & 7] = (__bf16)pv[r];
        }
      }
      // dV^T += dO^T P, one MFMA per slot; each slot also issues one pair of
      // Q^T reads, then (within a tile) one Q row fragment of the next unit
      // (2 DB = KC slots), and forms 16 / (2 DB) elements of dS = P (dP - D).
      // The first slot's product does not read dP: it runs through dP's
      // drain.  LDS reads complete in order, so the next unit's Q rows are
      // done once the dK products' waits for the later Q^T pairs are.
      constexpr int SE = 16 / (2 * DB);
      bf16x8 dsf[2];
      static_for<0, 2 * DB>([&](auto X) {
        constexpr int x = decltype(X)::value, hh = x / DB, d_ = x % DB;
        // dO^T pair x done (and D before it): the reads after it are the
        // later dO^T pairs, x Q^T pairs and, within a tile, x Q row
        // fragments; the wait counts the first two only, which is stricter
        // (the pair is an input, as the Q rows are above: only the asm
        // product reads it)
        constexpr int n = 4 * DB - 2 < 14 ? 4 * DB - 2 : 14;
        if constexpr (x == 0)
          asm volatile("s_waitcnt lgkmcnt(%4)"
                       : "+v"(d4[0]), "+v"(d4[1]), "+v"(d4[2]), "+v"(d4[3])
                       : "n"(n), "v"(olo[hh][d_]), "v"(ohi[hh][d_]));
        else
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(n), "v"(olo[hh][d_]), "v"(ohi[hh][d_]));
        const u32x4 wd = {olo[hh][d_][0], olo[hh][d_][1], ohi[hh][d_][0], ohi[hh][d_][1]};
        mfma_acc1(dva[d_], wd, pf[hh]);
        ds_rdtr<qo + (unsigned)hh * 32 * D>(qlo[hh][d_], ta.tr[0][d_]);
        ds_rdtr<qo + (unsigned)hh * 32 * D>(qhi[hh][d_], ta.tr[1][d_]);
        if constexpr (v + 1 < NU) read_q(ST, std::integral_constant<int, v + 1>{}, X);
        if constexpr (x == 0) qk_drain(dpa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < SE; ++q) {
          const int r = SE * x + q;
          dsf[r >> 3][r & 7] = (__bf16)(pv[r] * (dpa[r] - d4[r >> 2][r & 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // dK^T += Q^T dS in two halves of 16 query rows; between them the next
      // unit's LSE is read (its Q rows went out during the dV products)
      static_for<0, 2>([&](auto HH) {
        constexpr int hh = decltype(HH)::value;
        // Q^T pairs of this half done: after them come (within a tile) the
        // next unit's Q row fragment read with the half's last pair, then the
        // other half's pairs and fragments (first half) or the next unit's
        // LSE (second half)
        constexpr int F = v + 1 < NU ? 1 : 0;
        constexpr int n = hh == 0 ? F + DB * (2 + F) : 5 * F;
        if constexpr (DB == 4)
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(n), "v"(qlo[hh][0]), "v"(qhi[hh][0]), "v"(qlo[hh][1]),
                       "v"(qhi[hh][1]), "v"(qlo[hh][2]), "v"(qhi[hh][2]), "v"(qlo[hh][3]), "v"(qhi[hh][3]));
        else
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(n), "v"(qlo[hh][0]), "v"(qhi[hh][0]), "v"(qlo[hh][1]),
                       "v"(qhi[hh][1]));
        u32x4 wq[DB];
#pragma unroll
        for (int d_ = 0; d_ < DB; ++d_) wq[d_] = u32x4{qlo[hh][d_][0], qlo[hh][d_][1], qhi[hh][d_][0], qhi[hh][d_][1]};
        if constexpr (DB == 4) {
          mfma_acc4(dka[0], dka[1], dka[2], dka[3], wq[0], wq[1], wq[2], wq[3], dsf[hh]);
        } else {
#pragma unroll
          for (int d_ = 0; d_ < DB; ++d_) mfma_acc1(dka[d_], wq[d_], dsf[hh]);
        }
        if constexpr (hh == 0 && v + 1 < NU) read_l4(ST, std::integral_constant<int, v + 1>{});
      });
    });
  };
  if (total > 0) issue(0);
#pragma unroll
  for (int c = 0; c < KC; ++c) asm volatile("" : "+a"(kf[c]), "+a"(vf[c]));
  for (int it = 0; it < total; it += 2) {
    tile(it, std::integral_constant<int, 0>{});
    if (it + 1 < total) tile(it + 1, std::integral_constant<int, 1>{});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int d_ = 0; d_ < DB; ++d_) {
    mfma_acc_drain(dka[d_]);
    mfma_acc_drain(dva[d_]);
  }
  if (!k_ok) return;
  float* kp = a.dk + (int64_t)b * a.dk_sb + my_k * a.dk_ss + (int64_t)g * a.dk_sh;
  float* vp = a.dv + (int64_t)b * a.dv_sb + my_k * a.dv_ss + (int64_t)g * a.dv_sh;
#pragma unroll
  for (int d_ = 0; d_ < DB; ++d_)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 xk = {dka[d_][4 * j] * a.scale, dka[d_][4 * j + 1] * a.scale, dka[d_][4 * j + 2] * a.scale,
                        dka[d_][4 * j + 3] * a.scale};
      const f32x4 xv = {dva[d_][4 * j], dva[d_][4 * j + 1], dva[d_][4 * j + 2], dva[d_][4 * j + 3]};
      *(f32x4*)(kp + 32 * d_ + 8 * j + 4 * lg) = xk;
      *(f32x4*)(vp + 32 * d_ + 8 * j + 4 * lg) = xv;
    }
}

}  // namespace

hipError_t ra_launch_bwd(const RaBwdArgs& a, int d, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.nq;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a, d);
  const int64_t nqc = a.nsplit == 2 ? a.qc : a.nq;
  const dim3 gq((unsigned)((int64_t)a.nsplit * ((nqc + RA_BWD_BM - 1) / RA_BWD_BM) * a.Hq * a.B)), block(256);
  const dim3 gk((unsigned)(((a.N + RA_BWD_BM - 1) / RA_BWD_BM) * a.Hkv * a.B));
  if (d == 128) {
    hipLaunchKernelGGL(bwd_dq_kernel<128>, gq, block, 0, st, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, gk, block, 0, st, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<64>, gq, block, 0, st, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, gk, block, 0, st, a);
  }
  return hipGetLastError();
}
