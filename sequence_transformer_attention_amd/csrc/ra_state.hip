// ra_state.hip -- the HBM-bound kernels on the running state (o_acc, m, l).
//
// What is computed (glossary page "sequence parallelism transformers"):
// section "Ring Attention", item "Computation" -- a rank accumulates the
// result of every block it attends to, and the accumulation equals full
// attention; section "Implementation Considerations", item "Numerical
// Stability" -- the softmax normalisation travels with the partial result as
// a running maximum m and running sum l per query row.  The three kernels:
//   init      the empty state: o = 0, m = -inf, l = 0
//   merge     fold a second state into the first: m' = max(m, m_b),
//             w = e^{m - m'}, w_b = e^{m_b - m'} (0 for an empty side),
//             l' = w l + w_b l_b, o' = w o + w_b o_b
//   finalize  O = o / l, LSE = m + ln l
//
// Layout: o-type tensors [B, S, H, d] (d contiguous), row statistics [B, H, S].
// A workgroup takes RB consecutive sequence rows of one (batch, head).  Each
// row's d fp32 are one contiguous run, loaded with 16-byte loads by d / 4
// lanes; every lane issues all of its loads before the first use.  The row
// statistics of the RB rows are contiguous: lane i < RB of the workgroup
// loads and stores those of row i (coalesced), computes the row's factors
// once and hands them to the row's d / 4 lanes through LDS.  Index
// arithmetic is 32-bit apart from the final addresses (64-bit strides).
#include "ra_launch.h"

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

constexpr int kThreads = RA_STATE_THREADS;
constexpr int kUnroll = 4;  // rows per lane and workgroup: RB = kUnroll * kThreads / (d / 4)

// Position of this lane in a workgroup's block of rows: the workgroup's
// (batch, head) and first row s0, the lane's channel group c4 and its rows
// s0 + r0 + u * RSTEP (u < kUnroll).
template <int D>
struct RowBlock {
  static constexpr int ND4 = D / 4;             // lanes per row
  static constexpr int RSTEP = kThreads / ND4;  // rows per load instruction of the workgroup
  static constexpr int RB = kUnroll * RSTEP;    // rows per workgroup
  static_assert(RB <= kThreads, "one lane per row for the row statistics");
  int b, h, s0, c4, r0;
  __device__ __forceinline__ RowBlock(int H, int S) {
    const int nchunk = (S + RB - 1) / RB;
    const int bh = blockIdx.x / nchunk;  // workgroup-uniform
    b = bh / H;
    h = bh - b * H;
    s0 = (blockIdx.x - bh * nchunk) * RB;
    c4 = threadIdx.x % ND4;
    r0 = threadIdx.x / ND4;
  }
  __device__ __forceinline__ int row(int u) const { return r0 + u * RSTEP; }  // within the block
};

template <int D>
__global__ void __launch_bounds__(kThreads) finalize_kernel(RaFinArgs a) {
  using RB_t = RowBlock<D>;
  constexpr int RB = RB_t::RB;
  __shared__ float inv_s[RB];
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x;
  const float* ob = a.oacc + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
  f32x4 x[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.row(u);
    if (s < a.S) x[u] = *(const f32x4*)(ob + (int64_t)s * a.oa_ss);
  }
  if (tid < RB && rb.s0 + tid < a.S) {  // row statistics of row tid of the block
    const int s = rb.s0 + tid;
    const float lv = a.l[(int64_t)rb.b * a.l_sb + (int64_t)rb.h * a.l_sh + (int64_t)s * a.l_ss];
    inv_s[tid] = 1.f / lv;
    if (a.lse) {
      const float mv = a.m[(int64_t)rb.b * a.m_sb + (int64_t)rb.h * a.m_sh + (int64_t)s * a.m_ss];
      a.lse[(int64_t)rb.b * a.lse_sb + (int64_t)rb.h * a.lse_sh + (int64_t)s * a.lse_ss] = mv + logf(lv);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.row(u);
    if (s >= a.S) continue;
    const float inv = inv_s[rb.row(u)];
    const int64_t o = (int64_t)rb.b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)rb.h * a.o_sh + 4 * rb.c4;
    if (a.o_bf16)
      *(bf16x4*)((__bf16*)a.o + o) = bf16x4{(__bf16)(x[u][0] * inv), (__bf16)(x[u][1] * inv),
                                           (__bf16)(x[u][2] * inv), (__bf16)(x[u][3] * inv)};
    else
      *(f32x4*)((float*)a.o + o) = f32x4{x[u][0] * inv, x[u][1] * inv, x[u][2] * inv, x[u][3] * inv};
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) init_kernel(RaInitArgs a) {
  using RB_t = RowBlock<D>;
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x;
  float* ob = a.oacc + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.row(u);
    if (s < a.S) *(f32x4*)(ob + (int64_t)s * a.oa_ss) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < RB_t::RB && rb.s0 + tid < a.S) {
    const int s = rb.s0 + tid;
    a.m[(int64_t)rb.b * a.m_sb + (int64_t)rb.h * a.m_sh + (int64_t)s * a.m_ss] = -INFINITY;
    a.l[(int64_t)rb.b * a.l_sb + (int64_t)rb.h * a.l_sh + (int64_t)s * a.l_ss] = 0.f;
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(RaMergeArgs a) {
  using RB_t = RowBlock<D>;
  constexpr int RB = RB_t::RB;
  __shared__ float wa_s[RB], wb_s[RB];
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x;
  float* oa = a.oa + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
  const float* ob = a.ob + (int64_t)rb.b * a.ob_sb + (int64_t)rb.h * a.ob_sh + 4 * rb.c4;
  f32x4 xa[kUnroll], xb[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.row(u);
    if (s < a.S) {
      xa[u] = *(const f32x4*)(oa + (int64_t)s * a.oa_ss);
      xb[u] = *(const f32x4*)(ob + (int64_t)s * a.ob_ss);
    }
  }
  if (tid < RB && rb.s0 + tid < a.S) {  // row statistics of row tid of the block
    const int s = rb.s0 + tid;
    float* pma = a.ma + (int64_t)rb.b * a.ma_sb + (int64_t)rb.h * a.ma_sh + (int64_t)s * a.ma_ss;
    float* pla = a.la + (int64_t)rb.b * a.la_sb + (int64_t)rb.h * a.la_sh + (int64_t)s * a.la_ss;
    const float ma = *pma, la = *pla;
    const float mb = a.mb[(int64_t)rb.b * a.mb_sb + (int64_t)rb.h * a.mb_sh + (int64_t)s * a.mb_ss];
    const float lb = a.lb[(int64_t)rb.b * a.lb_sb + (int64_t)rb.h * a.lb_sh + (int64_t)s * a.lb_ss];
    const float mx = fmaxf(ma, mb);
    // an empty side (m = -inf) weighs 0; both empty stays empty
    const float wa = ma == -INFINITY ? 0.f : expf(ma - mx);
    const float wb = mb == -INFINITY ? 0.f : expf(mb - mx);
    wa_s[tid] = wa;
    wb_s[tid] = wb;
    *pma = mx;
    *pla = wa * la + wb * lb;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.row(u);
    if (s >= a.S) continue;
    const float wa = wa_s[rb.row(u)], wb = wb_s[rb.row(u)];
    *(f32x4*)(oa + (int64_t)s * a.oa_ss) =
        f32x4{wa * xa[u][0] + wb * xb[u][0], wa * xa[u][1] + wb * xb[u][1], wa * xa[u][2] + wb * xb[u][2],
              wa * xa[u][3] + wb * xb[u][3]};
  }
}

// Workgroups of a state kernel: B * H * ceil(S / RB).
inline dim3 state_grid(int B, int H, int S, int d) {
  return dim3((unsigned)ra_state_workgroups(B, H, S, d));
}

}  // namespace

int64_t ra_state_workgroups(int64_t B, int64_t H, int64_t S, int64_t d) {
  const int64_t rb = kUnroll * kThreads / (d / 4);
  return B * H * ((S + rb - 1) / rb);
}

hipError_t ra_launch_finalize(const RaFinArgs& a, hipStream_t st) {
  const dim3 grid = state_grid(a.B, a.H, a.S, a.d), block(kThreads);
  if (a.d == 128) hipLaunchKernelGGL(finalize_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(finalize_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_init(const RaInitArgs& a, hipStream_t st) {
  const dim3 grid = state_grid(a.B, a.H, a.S, a.d), block(kThreads);
  if (a.d == 128) hipLaunchKernelGGL(init_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(init_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t ra_launch_merge(const RaMergeArgs& a, hipStream_t st) {
  const dim3 grid = state_grid(a.B, a.H, a.S, a.d), block(kThreads);
  if (a.d == 128) hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}
