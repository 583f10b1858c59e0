// ra_f32.hip -- the fp32 attention kernel of libringattn (gfx950).
//
// What is computed (glossary page "sequence parallelism transformers"):
// section "Ring Attention", item "Computation" -- the rank's local queries
// against each key/value block in ring order, accumulated; section
// "Implementation Considerations", item "Numerical Stability" -- the softmax
// normalisation carried across blocks as a running max m and sum l per query
// row.  The same walk as the bf16 kernel (ring order, causal tile skipping,
// state in and out for ra_step), in fp32 FMA throughout: dot products,
// softmax, P V.
//
// A workgroup takes 64 query rows and splits every 64-key tile over
// RA_F32_KGROUPS = 4 key groups of waves (16 keys each).  In a group, each
// row belongs to LPR = D / 64 lanes of one wave (lanes l and l ^ 32 when
// D = 128), each holding 64 channels of the row's Q and O in registers, so
// the partial dot products of a key meet in one cross-lane swap.  The groups
// keep their own running state (m, l, O) for the same rows; after the last
// tile they merge it through LDS (m = max, l and O weighted by
// 2^(m_g - m), an empty group weighing 0) and group 0 writes the result.
// K and V tiles are staged in LDS by all threads and read by all lanes of a
// half-wave at the same address (broadcast).  Per group and tile: chunk max,
// rescale of O and l when it grows, exponentials, O += p V.
#include "ra_launch.h"
#include "ra_plan.h"

namespace {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ void __launch_bounds__(64 * (D / 64) * RA_F32_KGROUPS) attn_f32_kernel(RaAttnArgs a) {
  constexpr int BM = RA_F32_BM, BN = RA_F32_BN, KG = RA_F32_KGROUPS, CH = BN / KG;
  constexpr int LPR = D / 64, DL = D / LPR;  // lanes per row, channels per lane
  constexpr int GT = 64 * LPR, NT = GT * KG;  // threads per group, per workgroup
  constexpr int RS = D + 4;                   // floats per row in the merge buffer (16-byte aligned)
  constexpr int TILE_F = 2 * BN * D, MERGE_F = (KG - 1) * BM * RS;
  static_assert(DL == 64 && BM == 64 && CH == 16, "64 channels per lane, 64 rows, 16 keys per group");
  // K and V tiles during the walk; the groups' states for the merge after it
  __shared__ __attribute__((aligned(16))) float smem[TILE_F > MERGE_F ? TILE_F : MERGE_F];
  float* const Ks = smem;
  float* const Vs = smem + BN * D;
  const int tid = threadIdx.x;
  const int g = tid / GT, gt = tid % GT;  // key group, thread within it
  // row of the workgroup and channel half: rows 32 w .. 32 w + 31 in wave w
  // of the group when a row takes two lanes (l, l ^ 32), else row = lane
  const int lrow = LPR == 2 ? (gt >> 6) * 32 + (gt & 31) : gt;
  const int half = LPR == 2 ? (gt >> 5) & 1 : 0;
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
  const int qrow0 = (qt - chunk * nqt_c) * BM;  // the workgroup's first row within the chunk
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
  // running max m2 (log2 units of the scaled logits) and sum l of the
  // group's keys, the same in both lanes of a row; an incoming state (ra_step)
  // starts group 0, the others start empty
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) o[c] = 0.f;
  if (a.state_in && q_ok && g == 0) {
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
  const int j0 = g * CH;  // the group's keys in every tile
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
      // visible keys of this row in the tile: a prefix of lim; the group's
      // chunk is skipped when it lies past it (uniform per wave when it matters)
      const int lim = (int)ra_plan_visible_prefix(qpos, k0, nvalid, a.causal);
      if (j0 >= lim) continue;
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

  // Merge: groups 1 .. KG-1 leave (O, m, l) of each row in LDS (the tiles
  // are no longer read), group 0 folds them into its own.
  __syncthreads();
  if (g > 0) {
    float* slot = smem + ((g - 1) * BM + lrow) * RS;
#pragma unroll
    for (int c = 0; c < DL; c += 4) *(f32x4*)(slot + c0 + c) = f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]};
    if (half == 0) {
      slot[D] = m2;
      slot[D + 1] = lsum;
    }
  }
  __syncthreads();
  if (g > 0 || !q_ok) return;
#pragma unroll 1
  for (int gg = 1; gg < KG; ++gg) {
    const float* slot = smem + ((gg - 1) * BM + lrow) * RS;
    const float mo = slot[D], lo = slot[D + 1];
    const float mn = fmaxf(m2, mo);
    if (mn == -INFINITY) continue;  // neither has seen a key
    const float w0 = exp2f(m2 - mn), w1 = exp2f(mo - mn);  // 0 for an empty side
    lsum = lsum * w0 + lo * w1;
#pragma unroll
    for (int c = 0; c < DL; c += 4) {
      const f32x4 x = *(const f32x4*)(slot + c0 + c);
      o[c] = o[c] * w0 + x[0] * w1;
      o[c + 1] = o[c + 1] * w0 + x[1] * w1;
      o[c + 2] = o[c + 2] * w0 + x[2] * w1;
      o[c + 3] = o[c + 3] * w0 + x[3] * w1;
    }
    m2 = mn;
  }

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

hipError_t ra_launch_attn_f32(const RaAttnArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)(ra_query_tiles(a, RA_F32_BM) * a.Hq * a.B)), block(ra_f32_threads(d));
  if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}
