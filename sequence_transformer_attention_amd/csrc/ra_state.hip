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
// A workgroup takes RB consecutive sequence rows of one (batch, head): each
// row's d fp32 are one contiguous run (coalesced 16-byte loads; d / 4 lanes
// per row) and the row statistics of consecutive rows are contiguous.  Every
// lane issues all of its loads before the first use, so each workgroup keeps
// UNR x 16 bytes per lane in flight.  Index arithmetic is 32-bit apart from
// the final address (64-bit strides).
#include "ra_launch.h"

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

constexpr int kThreads = RA_STATE_THREADS;
constexpr int kUnroll = 4;  // rows per lane and workgroup (RB = kUnroll * kThreads / (d / 4))

// Position of this lane in a workgroup's block of rows: the workgroup's
// (batch, head) and first row, the lane's channel group c4 and its first row.
struct RowBlock {
  int b, h, s0, c4, r0, rstep;
};

template <int D>
__device__ __forceinline__ RowBlock row_block(int H, int S) {
  constexpr int ND4 = D / 4;                 // lanes per row
  constexpr int RSTEP = kThreads / ND4;      // rows per load instruction of the workgroup
  constexpr int RB = kUnroll * RSTEP;        // rows per workgroup
  const int nchunk = (S + RB - 1) / RB;
  const int bh = blockIdx.x / nchunk;        // scalar: once per workgroup
  RowBlock r;
  r.b = bh / H;
  r.h = bh - r.b * H;
  r.s0 = (blockIdx.x - bh * nchunk) * RB;
  r.c4 = threadIdx.x % ND4;
  r.r0 = threadIdx.x / ND4;
  r.rstep = RSTEP;
  return r;
}

template <int D>
__global__ void __launch_bounds__(kThreads) finalize_kernel(RaFinArgs a) {
  const RowBlock rb = row_block<D>(a.H, a.S);
  const float* ob = a.oacc + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
  const float* lb = a.l + (int64_t)rb.b * a.l_sb + (int64_t)rb.h * a.l_sh;
  f32x4 x[kUnroll];
  float lv[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.r0 + u * rb.rstep;
    if (s < a.S) {
      x[u] = *(const f32x4*)(ob + (int64_t)s * a.oa_ss);
      lv[u] = lb[(int64_t)s * a.l_ss];
    }
  }
  float mv[kUnroll];
  const bool lse = a.lse != nullptr && rb.c4 == 0;
  if (lse) {
    const float* mb = a.m + (int64_t)rb.b * a.m_sb + (int64_t)rb.h * a.m_sh;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = rb.s0 + rb.r0 + u * rb.rstep;
      if (s < a.S) mv[u] = mb[(int64_t)s * a.m_ss];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.r0 + u * rb.rstep;
    if (s >= a.S) continue;
    const float inv = 1.f / lv[u];
    const int64_t o = (int64_t)rb.b * a.o_sb + (int64_t)s * a.o_ss + (int64_t)rb.h * a.o_sh + 4 * rb.c4;
    if (a.o_bf16)
      *(bf16x4*)((__bf16*)a.o + o) = bf16x4{(__bf16)(x[u][0] * inv), (__bf16)(x[u][1] * inv),
                                           (__bf16)(x[u][2] * inv), (__bf16)(x[u][3] * inv)};
    else
      *(f32x4*)((float*)a.o + o) = f32x4{x[u][0] * inv, x[u][1] * inv, x[u][2] * inv, x[u][3] * inv};
    if (lse)
      a.lse[(int64_t)rb.b * a.lse_sb + (int64_t)rb.h * a.lse_sh + (int64_t)s * a.lse_ss] = mv[u] + logf(lv[u]);
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) init_kernel(RaInitArgs a) {
  const RowBlock rb = row_block<D>(a.H, a.S);
  float* ob = a.oacc + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.r0 + u * rb.rstep;
    if (s >= a.S) continue;
    *(f32x4*)(ob + (int64_t)s * a.oa_ss) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (rb.c4 == 0) {
      a.m[(int64_t)rb.b * a.m_sb + (int64_t)rb.h * a.m_sh + (int64_t)s * a.m_ss] = -INFINITY;
      a.l[(int64_t)rb.b * a.l_sb + (int64_t)rb.h * a.l_sh + (int64_t)s * a.l_ss] = 0.f;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(RaMergeArgs a) {
  const RowBlock rb = row_block<D>(a.H, a.S);
  float* oa = a.oa + (int64_t)rb.b * a.oa_sb + (int64_t)rb.h * a.oa_sh + 4 * rb.c4;
  const float* ob = a.ob + (int64_t)rb.b * a.ob_sb + (int64_t)rb.h * a.ob_sh + 4 * rb.c4;
  float* ma = a.ma + (int64_t)rb.b * a.ma_sb + (int64_t)rb.h * a.ma_sh;
  float* la = a.la + (int64_t)rb.b * a.la_sb + (int64_t)rb.h * a.la_sh;
  const float* mb = a.mb + (int64_t)rb.b * a.mb_sb + (int64_t)rb.h * a.mb_sh;
  const float* lb = a.lb + (int64_t)rb.b * a.lb_sb + (int64_t)rb.h * a.lb_sh;
  f32x4 xa[kUnroll], xb[kUnroll];
  float mav[kUnroll], mbv[kUnroll], lav[kUnroll], lbv[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.r0 + u * rb.rstep;
    if (s < a.S) {
      xa[u] = *(const f32x4*)(oa + (int64_t)s * a.oa_ss);
      xb[u] = *(const f32x4*)(ob + (int64_t)s * a.ob_ss);
      mav[u] = ma[(int64_t)s * a.ma_ss];
      mbv[u] = mb[(int64_t)s * a.mb_ss];
      lav[u] = la[(int64_t)s * a.la_ss];
      lbv[u] = lb[(int64_t)s * a.lb_ss];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int s = rb.s0 + rb.r0 + u * rb.rstep;
    if (s >= a.S) continue;
    const float mx = fmaxf(mav[u], mbv[u]);
    // an empty side (m = -inf) weighs 0; both empty stays empty
    const float wa = mav[u] == -INFINITY ? 0.f : expf(mav[u] - mx);
    const float wb = mbv[u] == -INFINITY ? 0.f : expf(mbv[u] - mx);
    *(f32x4*)(oa + (int64_t)s * a.oa_ss) =
        f32x4{wa * xa[u][0] + wb * xb[u][0], wa * xa[u][1] + wb * xb[u][1], wa * xa[u][2] + wb * xb[u][2],
              wa * xa[u][3] + wb * xb[u][3]};
    if (rb.c4 == 0) {
      ma[(int64_t)s * a.ma_ss] = mx;
      la[(int64_t)s * a.la_ss] = wa * lav[u] + wb * lbv[u];
    }
  }
}

// Workgroups of a state kernel: B * H * ceil(S / RB).
inline dim3 state_grid(int B, int H, int S, int d) {
  const int rb = kUnroll * kThreads / (d / 4);
  return dim3((unsigned)((int64_t)B * H * ((S + rb - 1) / rb)));
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
