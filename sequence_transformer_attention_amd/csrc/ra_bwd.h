// ra_bwd.h -- argument block and launchers of the backward kernels (internal
// to libringattn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Backward of one rank's share (contiguous blocks, bf16 inputs):
//   q, o, dout: [B, nq, Hq, d] bf16, the rank's local rows (positions q_off..)
//   k, v:       [B, N, Hkv, d] bf16, the whole sequence (row = position)
//   lse:        [B, Hq, nq] fp32, natural log, from the forward
//   delta:      [B, Hq, nq] fp32 workspace, written by the prep kernel with
//               D_i = <dO_i, O_i>
//   dq:         [B, nq, Hq, d] fp32 out
//   dk, dv:     [B, N, Hkv, d] fp32 out: this rank's contribution
// Strides are in elements ([b, s, h] order for the 4-d tensors, [b, h, s]
// for the row statistics).
struct RaBwdArgs {
  const void* q; int64_t q_sb, q_ss, q_sh;
  const void* k; int64_t k_sb, k_ss, k_sh;
  const void* v; int64_t v_sb, v_ss, v_sh;
  const void* o; int64_t o_sb, o_ss, o_sh;
  const void* dout; int64_t do_sb, do_ss, do_sh;
  const float* lse; int64_t lse_sb, lse_sh, lse_ss;
  float* delta; int64_t de_sb, de_sh, de_ss;
  float* dq; int64_t dq_sb, dq_ss, dq_sh;
  float* dk; int64_t dk_sb, dk_ss, dk_sh;
  float* dv; int64_t dv_sb, dv_ss, dv_sh;
  int32_t B, Hq, Hkv, nq;
  int64_t N, nb, q_off;
  int32_t P, rank, causal;
  // query split of the load-balanced share (nsplit = 2): local rows
  // [0, qc) at positions q_off.. (ring rank `rank` over 2P chunks of qc
  // keys), rows [qc, 2qc) at positions q_off2.. (ring rank rank2); nsplit = 1:
  // one block of nq rows, P blocks of nb keys
  int32_t nsplit, rank2;
  int64_t qc, q_off2;
  // keys at positions >= kv_end are visible to no query (an explicitly
  // padded sequence; N otherwise)
  int64_t kv_end;
  float c;       // softmax scale * log2(e)
  float scale;   // softmax scale
};

// Rows of a workgroup: queries of the dQ kernel, keys of the dK/dV kernel.
constexpr int RA_BWD_BM = 128, RA_BWD_BN = 64;
constexpr int RA_BWD_THREADS = 256;  // threads per workgroup of every backward kernel

hipError_t ra_launch_bwd(const RaBwdArgs& a, int d, hipStream_t s);
