// ra_launch.h -- kernel argument blocks and launchers (internal to libringattn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Attention over one or more key/value blocks for a query block.
//   ring == 0: one step, keys at global kv_off.., k/v point at the block.
//   ring == 1: P steps in ring order from `rank`; k/v point at the whole
//              sequence [B, P*nkv, Hkv, d]; q_off = rank * nkv.
//   nsplit:    2 = the local rows are two chunks of qc rows: rows [0, qc)
//              at global positions q_off.. (ring order from rank), rows
//              [qc, 2 qc) at q_off2.. (ring order from rank2); otherwise one
//              block of nq rows at q_off.. .  Query tiles never straddle the
//              chunks.
//   kv_end:    keys at global positions >= kv_end are not visible (the
//              valid length of an explicitly padded sequence; the end of the
//              block or sequence otherwise).
//   state_in:  1 = start from (oacc, m, l); 0 = start from the empty state.
//   out_state: 1 = write (oacc, m, l) back; 0 = write normalised o (+ lse).
struct RaAttnArgs {
  const void* q; int64_t q_sb, q_ss, q_sh;
  const void* k; int64_t k_sb, k_ss, k_sh;
  const void* v; int64_t v_sb, v_ss, v_sh;
  int32_t B, Hq, Hkv, nq;
  int64_t nkv;               // block length
  int64_t q_off, kv_off;
  int32_t ring, P, rank, causal;
  float c;                   // softmax scale * log2(e)
  int32_t state_in, out_state;
  float* oacc; int64_t oa_sb, oa_ss, oa_sh;
  float* m; int64_t m_sb, m_sh, m_ss;
  float* l; int64_t l_sb, l_sh, l_ss;
  void* o; int64_t o_sb, o_ss, o_sh; int32_t o_bf16;
  float* lse; int64_t lse_sb, lse_sh, lse_ss;
  int32_t nsplit, rank2; int64_t qc, q_off2;
  int64_t kv_end;
};

// O = oacc / l (to o, bf16 or fp32, or in place), LSE = m + ln l (optional).
struct RaFinArgs {
  const float* oacc; int64_t oa_sb, oa_ss, oa_sh;
  const float* m; int64_t m_sb, m_sh, m_ss;
  const float* l; int64_t l_sb, l_sh, l_ss;
  void* o; int64_t o_sb, o_ss, o_sh; int32_t o_bf16;
  float* lse; int64_t lse_sb, lse_sh, lse_ss;
  int32_t B, H, S, d;
};

// oacc = 0, m = -inf, l = 0.
struct RaInitArgs {
  float* oacc; int64_t oa_sb, oa_ss, oa_sh;
  float* m; int64_t m_sb, m_sh, m_ss;
  float* l; int64_t l_sb, l_sh, l_ss;
  int32_t B, H, S, d;
};

// (oa, ma, la) <- merge((oa, ma, la), (ob, mb, lb)), in place.
struct RaMergeArgs {
  float* oa; int64_t oa_sb, oa_ss, oa_sh;
  float* ma; int64_t ma_sb, ma_sh, ma_ss;
  float* la; int64_t la_sb, la_sh, la_ss;
  const float* ob; int64_t ob_sb, ob_ss, ob_sh;
  const float* mb; int64_t mb_sb, mb_sh, mb_ss;
  const float* lb; int64_t lb_sb, lb_sh, lb_ss;
  int32_t B, H, S, d;
};

// Threads per workgroup of the state kernels (init, merge, finalize), and
// their workgroup count for a [B, S, H, d] state (d = 64 or 128).
constexpr int RA_STATE_THREADS = 512;
int64_t ra_state_workgroups(int64_t B, int64_t H, int64_t S, int64_t d);

// Tile shape of the attention kernels (query rows per workgroup, keys per tile).
constexpr int RA_BF16_BM = 256, RA_BF16_BN = 64;
constexpr int RA_F32_BM = 64, RA_F32_BN = 64;
// Threads per workgroup of the attention kernels.  The fp32 one splits each
// key tile over RA_F32_KGROUPS groups of 64 threads per 64 channels of the
// head dimension: ra_f32_threads(d), at most RA_F32_THREADS.
constexpr int RA_BF16_THREADS = 256, RA_F32_KGROUPS = 4, RA_F32_THREADS = 128 * RA_F32_KGROUPS;
constexpr int ra_f32_threads(int d) { return 64 * (d / 64) * RA_F32_KGROUPS; }

// Query tiles of a launch: per chunk ceil(rows / BM), times the chunk count.
inline int64_t ra_query_tiles(const RaAttnArgs& a, int bm) {
  const int64_t rows = a.nsplit == 2 ? a.qc : a.nq;
  return (a.nsplit == 2 ? 2 : 1) * ((rows + bm - 1) / bm);
}

hipError_t ra_launch_attn_bf16(const RaAttnArgs& a, int d, hipStream_t s);
hipError_t ra_launch_attn_f32(const RaAttnArgs& a, int d, hipStream_t s);
hipError_t ra_launch_finalize(const RaFinArgs& a, hipStream_t s);
hipError_t ra_launch_init(const RaInitArgs& a, hipStream_t s);
hipError_t ra_launch_merge(const RaMergeArgs& a, hipStream_t s);
