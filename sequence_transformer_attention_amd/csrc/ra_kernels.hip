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
// bf16 path (attn_bf16_kernel), one workgroup = 4 waves = 128 query rows of
// one head; each wave owns 32 query rows.  Per key tile of 64 keys:
//   S^T (keys x queries) = K Q^T   v_mfma_f32_32x32x16_bf16, K from LDS (A),
//                                  Q fragment in VGPRs for the whole kernel (B)
//   online softmax                 the accumulator layout puts one query per
//                                  lane (lane & 31) and 32 of its 64 keys in
//                                  that lane's registers; the other 32 sit in
//                                  lane ^ 32, so the row max needs one
//                                  cross-lane exchange and the rescale factor
//                                  is a per-lane scalar
//   O^T (channels x queries) += V^T P^T   P^T goes from the S^T accumulator
//                                  registers straight into the B operand
//                                  (bf16, round to nearest even); V^T is
//                                  staged transposed in LDS for the A operand
// K and V tiles move HBM -> VGPR (128-bit loads, prefetched one tile ahead)
// -> LDS (double-buffered, one barrier per tile).  Logits are scaled in fp32
// (never folded into bf16 Q); exponentials are base 2 with the scale folded
// into one FMA: p = exp2(s * scale * log2(e) - m2), m2 the running max in
// log2 units.
#include "ra_launch.h"
#include "ra_plan.h"

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

__device__ __forceinline__ unsigned bf16_at(const u32x4& v, int e) {
  unsigned w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(RaAttnArgs a) {
  constexpr int BM = RA_BF16_BM, BN = RA_BF16_BN, NT = 256;
  constexpr int KROW = D + 8;   // bf16 per K row in LDS: 16-byte pad, rows shift 4 banks
  constexpr int VROW = BN + 4;  // bf16 per V^T row in LDS: 8-byte pad, rows shift 2 banks
  constexpr int KSZ = BN * KROW, VSZ = D * VROW, STAGE = KSZ + VSZ;
  constexpr int NKC = BN * D / 8 / NT;     // 16-byte K chunks per thread per tile
  constexpr int NVG = (BN / 4) * (D / 8);  // V groups of 4 keys x 8 channels
  static_assert(NKC * NT * 8 == BN * D, "K tile split");
  static_assert(NVG <= NT, "V tile split");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  auto step_kv_off = [&](int s) -> int64_t {
    return a.ring ? ra_plan_ring_block(a.P, a.rank, s) * a.nkv : a.kv_off;
  };
  auto step_row0 = [&](int s) -> int64_t {
    return a.ring ? ra_plan_ring_block(a.P, a.rank, s) * a.nkv : 0;
  };
  auto step_tiles = [&](int s) -> int {
    return (int)ra_plan_key_tiles(q0_wg, nq_wg, step_kv_off(s), a.nkv, a.causal, BN);
  };

  u32x4 kreg[NKC];
  u32x4 vreg[4];
  const int vga = tid % (BN / 4), vdc = tid / (BN / 4);

  auto load_tile = [&](int s, int u) {
    const int64_t r0 = step_row0(s) + (int64_t)u * BN;
    const int64_t left = a.nkv - (int64_t)u * BN;
    const int nvalid = left < BN ? (int)left : BN;
    const __bf16* kb = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh + r0 * a.k_ss;
    const __bf16* vb = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh + r0 * a.v_ss;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int id = tid + i * NT, row = id / (D / 8), ch = id % (D / 8);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < nvalid) w = *(const u32x4*)(kb + (int64_t)row * a.k_ss + ch * 8);
      kreg[i] = w;
    }
    if (tid < NVG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * vga + i;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (row < nvalid) w = *(const u32x4*)(vb + (int64_t)row * a.v_ss + vdc * 8);
        vreg[i] = w;
      }
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* Ks = smem + buf * STAGE;
    __bf16* Vt = Ks + KSZ;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int id = tid + i * NT, row = id / (D / 8), ch = id % (D / 8);
      *(u32x4*)(Ks + row * KROW + ch * 8) = kreg[i];
    }
    if (tid < NVG) {
      // 4 keys x 8 channels -> V^T rows 8vdc..8vdc+7, keys 4vga..4vga+3
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x2 w;
        w[0] = bf16_at(vreg[0], e) | (bf16_at(vreg[1], e) << 16);
        w[1] = bf16_at(vreg[2], e) | (bf16_at(vreg[3], e) << 16);
        *(u32x2*)(Vt + (8 * vdc + e) * VROW + 4 * vga) = w;
      }
    }
  };

  auto compute = [&](int s, int u, int buf) {
    const __bf16* Ks = smem + buf * STAGE;
    const __bf16* Vt = Ks + KSZ;
    const int64_t k0 = step_kv_off(s) + (int64_t)u * BN;
    const int64_t left = a.nkv - (int64_t)u * BN;
    const int nvalid = left < BN ? (int)left : BN;
    const int64_t q0w = a.q_off + qrow_w;
    const int nqw = min(32, a.nq - qrow_w);
    const int cls = ra_plan_class(q0w, nqw, k0, nvalid, a.causal);
    if (cls == RA_CLASS_SKIP) return;  // wave-uniform: no visible key for these rows
    const bool need_mask = cls == RA_CLASS_PARTIAL || nvalid < BN;

    f32x16 sacc[BN / 32];
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb) {
      sacc[bb] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 kf = *(const bf16x8*)(Ks + (32 * bb + lr) * KROW + 16 * c + 8 * lg);
        sacc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc[bb], 0, 0, 0);
      }
    }
    if (need_mask) {
      const int64_t qpos = q0w + lr;
#pragma unroll
      for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kvi = 32 * bb + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (kvi >= nvalid || (a.causal && k0 + kvi > qpos)) sacc[bb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[bb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m2, mx * a.c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no key yet: keep p = 0, alpha = 0
    const float alpha = fast_exp2(m2 - m_use);

    bf16x8 pf[BN / 32][2];
    float psum = 0.f;
#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[bb][r], a.c, -m_use));
        psum += p;
        pf[bb][r >> 3][r & 7] = (__bf16)p;
      }
    lsum = lsum * alpha + psum;
    m2 = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

#pragma unroll
    for (int bb = 0; bb < BN / 32; ++bb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const __bf16* vp = Vt + (32 * db + lr) * VROW + 32 * bb + 16 * hh + 4 * lg;
          const bf16x4 lo = *(const bf16x4*)vp;
          const bf16x4 hi = *(const bf16x4*)(vp + 8);
          const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[bb][hh], o[db], 0, 0, 0);
        }
  };

  // Flat loop over (step, tile) in ring order; tile i+1 is fetched into
  // registers while tile i is computed from LDS buffer i & 1.
  int s = 0;
  while (s < nsteps && step_tiles(s) == 0) ++s;
  int u = 0, it = 0;
  if (s < nsteps) load_tile(s, 0);
  while (s < nsteps) {
    const int nt = step_tiles(s);
    store_tile(it & 1);
    __syncthreads();
    int s2 = s, u2 = u + 1;
    if (u2 >= nt) {
      u2 = 0;
      ++s2;
      while (s2 < nsteps && step_tiles(s2) == 0) ++s2;
    }
    if (s2 < nsteps) load_tile(s2, u2);
    compute(s, u, it & 1);
    s = s2;
    u = u2;
    ++it;
  }

  // Epilogue: the two halves of each row sum live in lanes lr and lr + 32.
  const float ltot = lsum + __shfl_xor(lsum, 32);
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
  const dim3 grid((unsigned)((int64_t)nqt * a.Hq * a.B)), block(256);
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
