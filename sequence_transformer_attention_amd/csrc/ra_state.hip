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
// Layout: o-type tensors [B, S, H, d] (d contiguous, any strides), row
// statistics [B, H, S].  A workgroup takes a block of RB rows of one batch:
// HB heads x RB / HB sequence rows, rows in (sequence row, head) order.
// When the heads of a sequence row are adjacent in every o-type tensor of
// the call (the plain [B, S, H, d] layout) and H is a multiple of 8, HB = 8
// and a block is RB / 8 runs of 8 d fp32 (4 KiB at d = 128) in each
// tensor; otherwise HB = 1 (RB sequence rows of one head, contiguous in the
// row statistics and in a [B, H, S, d] buffer).  Measured on 131072 rows of
// d = 128 with the state in HBM, the 8-head blocks move 4-9 % more bytes per
// second than the one-head blocks of the same size in all three kernels.
// Each row's d fp32 are loaded with 16-byte loads by d / 4 lanes; every
// lane issues all of its loads before the first use.  Lane j < RB of the
// workgroup loads and stores the row statistics of one row (consecutive
// lanes, consecutive sequence rows of one head), computes the row's factors
// once and hands them to the row's d / 4 lanes through LDS.  Index
// arithmetic is 32-bit apart from the final addresses (64-bit strides).
// The finalize reads o_acc and writes O with non-temporal accesses: the
// state is read once and the output is not read back here, and with the
// state in HBM the kernel moves about 16 % more bytes per second that way
// (the same from the last-level cache).  The merge keeps cached accesses:
// its result is the next step's input, and from the cache the non-temporal
// form ran 7-13 % slower.
#include "ra_launch.h"

#include <initializer_list>

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

constexpr int kThreads = RA_STATE_THREADS;
constexpr int kUnroll = 4;  // rows per lane: RB = kUnroll * kThreads / (d / 4)
constexpr int kHeads = 8;   // heads per block when the heads of a row are adjacent

// A workgroup's block of rows: HB heads x SB sequence rows of one batch.
// Row i of the block is head h0 + i % HB, sequence row s0 + i / HB.  This
// lane's channel group c4 and its rows row(u) = r0 + u * RSTEP (u < kUnroll)
// of the block; the lane of row statistic j takes row stat_row(j) = head
// j / SB, sequence row j % SB.
template <int D, int HB>
struct RowBlock {
  static constexpr int ND4 = D / 4;             // lanes per row
  static constexpr int RSTEP = kThreads / ND4;  // rows per load instruction of the workgroup
  static constexpr int RB = kUnroll * RSTEP;    // rows per workgroup
  static constexpr int SB = RB / HB;            // sequence rows per workgroup
  static_assert(RB <= kThreads, "one lane per row for the row statistics");
  static_assert(RB % HB == 0, "whole sequence rows per block");
  int H, S, b, h0, s0, c4, r0;
  __device__ __forceinline__ RowBlock(int H_, int S_) : H(H_), S(S_) {
    const int nchunk = (S + SB - 1) / SB, nhg = (H + HB - 1) / HB;
    const int bg = blockIdx.x / nchunk;  // workgroup-uniform
    b = bg / nhg;
    h0 = (bg - b * nhg) * HB;
    s0 = (blockIdx.x - bg * nchunk) * SB;
    c4 = threadIdx.x % ND4;
    r0 = threadIdx.x / ND4;
  }
  __device__ __forceinline__ int row(int u) const { return r0 + u * RSTEP; }
  __device__ __forceinline__ int stat_row(int j) const { return (j % SB) * HB + j / SB; }
  // head and sequence row of row i of the block; false past the edges
  __device__ __forceinline__ bool at(int i, int& h, int& s) const {
    h = h0 + i % HB;
    s = s0 + i / HB;
    return h < H && s < S;
  }
};

__device__ __forceinline__ int64_t off3(int b, int h, int s, int64_t sb, int64_t sh, int64_t ss) {
  return (int64_t)b * sb + (int64_t)h * sh + (int64_t)s * ss;
}

template <int D, int HB>
__global__ void __launch_bounds__(kThreads) finalize_kernel(RaFinArgs a) {
  using RB_t = RowBlock<D, HB>;
  constexpr int RB = RB_t::RB;
  __shared__ float inv_s[RB];
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x, b = rb.b;
  f32x4 x[kUnroll];
  bool ok[kUnroll];
  int64_t oo[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    int h, s;
    ok[u] = rb.at(rb.row(u), h, s);
    oo[u] = off3(b, h, s, a.o_sb, a.o_sh, a.o_ss) + 4 * rb.c4;
    if (ok[u]) x[u] = __builtin_nontemporal_load((const f32x4*)(a.oacc + off3(b, h, s, a.oa_sb, a.oa_sh, a.oa_ss) + 4 * rb.c4));
  }
  const int j = rb.stat_row(tid);
  int h, s;
  if (tid < RB && rb.at(j, h, s)) {  // row statistics of row j of the block
    const float lv = a.l[off3(b, h, s, a.l_sb, a.l_sh, a.l_ss)];
    inv_s[j] = 1.f / lv;
    if (a.lse)
      a.lse[off3(b, h, s, a.lse_sb, a.lse_sh, a.lse_ss)] = a.m[off3(b, h, s, a.m_sb, a.m_sh, a.m_ss)] + logf(lv);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (!ok[u]) continue;
    const float inv = inv_s[rb.row(u)];
    if (a.o_bf16)
      __builtin_nontemporal_store(bf16x4{(__bf16)(x[u][0] * inv), (__bf16)(x[u][1] * inv),
                                         (__bf16)(x[u][2] * inv), (__bf16)(x[u][3] * inv)},
                                  (bf16x4*)((__bf16*)a.o + oo[u]));
    else
      __builtin_nontemporal_store(f32x4{x[u][0] * inv, x[u][1] * inv, x[u][2] * inv, x[u][3] * inv},
                                  (f32x4*)((float*)a.o + oo[u]));
  }
}

template <int D, int HB>
__global__ void __launch_bounds__(kThreads) init_kernel(RaInitArgs a) {
  using RB_t = RowBlock<D, HB>;
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x, b = rb.b;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    int h, s;
    if (rb.at(rb.row(u), h, s))
      *(f32x4*)(a.oacc + off3(b, h, s, a.oa_sb, a.oa_sh, a.oa_ss) + 4 * rb.c4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int h, s;
  if (tid < RB_t::RB && rb.at(rb.stat_row(tid), h, s)) {
    a.m[off3(b, h, s, a.m_sb, a.m_sh, a.m_ss)] = -INFINITY;
    a.l[off3(b, h, s, a.l_sb, a.l_sh, a.l_ss)] = 0.f;
  }
}

template <int D, int HB>
__global__ void __launch_bounds__(kThreads) merge_kernel(RaMergeArgs a) {
  using RB_t = RowBlock<D, HB>;
  constexpr int RB = RB_t::RB;
  __shared__ float wa_s[RB], wb_s[RB];
  const RB_t rb(a.H, a.S);
  const int tid = threadIdx.x, b = rb.b;
  f32x4 xa[kUnroll], xb[kUnroll];
  bool ok[kUnroll];
  int64_t oa[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    int h, s;
    ok[u] = rb.at(rb.row(u), h, s);
    oa[u] = off3(b, h, s, a.oa_sb, a.oa_sh, a.oa_ss) + 4 * rb.c4;
    if (ok[u]) {
      xa[u] = *(const f32x4*)(a.oa + oa[u]);
      xb[u] = *(const f32x4*)(a.ob + off3(b, h, s, a.ob_sb, a.ob_sh, a.ob_ss) + 4 * rb.c4);
    }
  }
  const int j = rb.stat_row(tid);
  int h, s;
  if (tid < RB && rb.at(j, h, s)) {  // row statistics of row j of the block
    float* pma = a.ma + off3(b, h, s, a.ma_sb, a.ma_sh, a.ma_ss);
    float* pla = a.la + off3(b, h, s, a.la_sb, a.la_sh, a.la_ss);
    const float ma = *pma, la = *pla;
    const float mb = a.mb[off3(b, h, s, a.mb_sb, a.mb_sh, a.mb_ss)];
    const float lb = a.lb[off3(b, h, s, a.lb_sb, a.lb_sh, a.lb_ss)];
    const float mx = fmaxf(ma, mb);
    // an empty side (m = -inf) weighs 0; both empty stays empty
    const float wa = ma == -INFINITY ? 0.f : expf(ma - mx);
    const float wb = mb == -INFINITY ? 0.f : expf(mb - mx);
    wa_s[j] = wa;
    wb_s[j] = wb;
    *pma = mx;
    *pla = wa * la + wb * lb;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (!ok[u]) continue;
    const float wa = wa_s[rb.row(u)], wb = wb_s[rb.row(u)];
    *(f32x4*)(a.oa + oa[u]) = f32x4{wa * xa[u][0] + wb * xb[u][0], wa * xa[u][1] + wb * xb[u][1],
                                    wa * xa[u][2] + wb * xb[u][2], wa * xa[u][3] + wb * xb[u][3]};
  }
}

// Workgroups of a state kernel with HB heads per block.
template <int HB>
int64_t workgroups(int64_t B, int64_t H, int64_t S, int64_t d) {
  const int64_t sb = kUnroll * kThreads / (d / 4) / HB;
  return B * ((H + HB - 1) / HB) * ((S + sb - 1) / sb);
}

// The 8-head blocks: H a multiple of 8 and, in every o-type tensor of the
// call, head stride d.
inline bool head_blocks(int64_t H, int64_t d, std::initializer_list<int64_t> head_strides) {
  if (H % kHeads) return false;
  for (int64_t x : head_strides)
    if (x != d) return false;
  return true;
}

// Launch K<D, kHeads> or K<D, 1> over the state's blocks.
template <typename A>
hipError_t launch(void (*k8)(A), void (*k1)(A), bool heads8, const A& a, hipStream_t st) {
  if (heads8)
    hipLaunchKernelGGL(k8, dim3((unsigned)workgroups<kHeads>(a.B, a.H, a.S, a.d)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k1, dim3((unsigned)workgroups<1>(a.B, a.H, a.S, a.d)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// The larger grid of the two block shapes: the one-head blocks (8-head
// blocks are used only when 8 divides H, and then need no more).
int64_t ra_state_workgroups(int64_t B, int64_t H, int64_t S, int64_t d) { return workgroups<1>(B, H, S, d); }

hipError_t ra_launch_finalize(const RaFinArgs& a, hipStream_t st) {
  const bool h8 = head_blocks(a.H, a.d, {a.oa_sh, a.o_sh});
  if (a.d == 128) return launch(finalize_kernel<128, kHeads>, finalize_kernel<128, 1>, h8, a, st);
  return launch(finalize_kernel<64, kHeads>, finalize_kernel<64, 1>, h8, a, st);
}

hipError_t ra_launch_init(const RaInitArgs& a, hipStream_t st) {
  const bool h8 = head_blocks(a.H, a.d, {a.oa_sh});
  if (a.d == 128) return launch(init_kernel<128, kHeads>, init_kernel<128, 1>, h8, a, st);
  return launch(init_kernel<64, kHeads>, init_kernel<64, 1>, h8, a, st);
}

hipError_t ra_launch_merge(const RaMergeArgs& a, hipStream_t st) {
  const bool h8 = head_blocks(a.H, a.d, {a.oa_sh, a.ob_sh});
  if (a.d == 128) return launch(merge_kernel<128, kHeads>, merge_kernel<128, 1>, h8, a, st);
  return launch(merge_kernel<64, kHeads>, merge_kernel<64, 1>, h8, a, st);
}
