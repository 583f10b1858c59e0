// ra_api.cpp -- the C ABI of libringattn: argument checks, planning, launches.
//
// Every entry point validates all of its arguments on the host first and only
// then touches the HIP runtime, so a bad call never reaches the GPU.  The
// operations are those of the glossary page "sequence parallelism
// transformers", section "Ring Attention" (items "Ring Communication" and
// "Computation"); the argument and layout rules are documented in
// include/libringattn.h.
#include "../../include/libringattn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <mutex>

#include "ra_bwd.h"
#include "ra_launch.h"
#include "ra_plan.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return RA_OK;
}

size_t esize(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }

bool dtype_valid(int32_t dt) { return dt == RA_BF16 || dt == RA_F32; }

// A [B, S, H, d] tensor: stride[3] == 1, 16-byte aligned data and strides of
// every dimension that has more than one entry.
int check_bshd(const ra_tensor* t, const char* name) {
  if (!t) return fail(RA_E_NULL, "%s is NULL", name);
  if (!dtype_valid(t->dtype)) return fail(RA_E_DTYPE, "%s: unknown dtype %d", name, (int)t->dtype);
  int64_t numel = 1;
  for (int i = 0; i < 4; ++i) {
    if (t->shape[i] < 0) return fail(RA_E_SHAPE, "%s: negative shape[%d]", name, i);
    numel *= t->shape[i];
  }
  if (numel == 0) return RA_OK;
  if (!t->data) return fail(RA_E_NULL, "%s->data is NULL", name);
  if (t->stride[3] != 1 && t->shape[3] > 1)
    return fail(RA_E_LAYOUT, "%s: stride[3] must be 1 (got %lld)", name, (long long)t->stride[3]);
  if (((uintptr_t)t->data) % 16 != 0) return fail(RA_E_LAYOUT, "%s: data not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i) {
    if (t->shape[i] <= 1) continue;
    if (t->stride[i] < 0) return fail(RA_E_LAYOUT, "%s: negative stride[%d]", name, i);
    if ((t->stride[i] * (int64_t)esize(t->dtype)) % 16 != 0)
      return fail(RA_E_LAYOUT, "%s: stride[%d] * element size is not a multiple of 16 bytes", name, i);
  }
  return RA_OK;
}

// A per-row statistic [B, H, S, 1], fp32.
int check_rows(const ra_tensor* t, const char* name, int64_t B, int64_t H, int64_t S) {
  if (!t) return fail(RA_E_NULL, "%s is NULL", name);
  if (t->dtype != RA_F32) return fail(RA_E_DTYPE, "%s must be fp32", name);
  if (t->shape[0] != B || t->shape[1] != H || t->shape[2] != S || t->shape[3] != 1)
    return fail(RA_E_SHAPE, "%s: shape must be [%lld, %lld, %lld, 1], got [%lld, %lld, %lld, %lld]", name,
                (long long)B, (long long)H, (long long)S, (long long)t->shape[0], (long long)t->shape[1],
                (long long)t->shape[2], (long long)t->shape[3]);
  if (B * H * S == 0) return RA_OK;
  if (!t->data) return fail(RA_E_NULL, "%s->data is NULL", name);
  if (((uintptr_t)t->data) % 4 != 0) return fail(RA_E_LAYOUT, "%s: data not 4-byte aligned", name);
  for (int i = 0; i < 3; ++i)
    if (t->stride[i] < 0) return fail(RA_E_LAYOUT, "%s: negative stride[%d]", name, i);
  return RA_OK;
}

bool same_shape(const ra_tensor* a, const ra_tensor* b) {
  for (int i = 0; i < 4; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

float resolve_scale(const ra_opts* opts, int64_t d) {
  if (opts && opts->scale > 0.f && isfinite(opts->scale)) return opts->scale;
  return (float)(1.0 / sqrt((double)d));
}

hipStream_t stream_of(const ra_opts* opts) { return opts ? (hipStream_t)opts->stream : nullptr; }

// q [B, Nq, Hq, d] and k, v [B, Nkv, Hkv, d]: dtypes, shapes, head_dim.
int check_qkv(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const char* kn, const char* vn) {
  int e;
  if ((e = check_bshd(q, "q")) || (e = check_bshd(k, kn)) || (e = check_bshd(v, vn))) return e;
  if (q->dtype != k->dtype || q->dtype != v->dtype)
    return fail(RA_E_DTYPE, "q, %s and %s must have the same dtype", kn, vn);
  if (!same_shape(k, v)) return fail(RA_E_SHAPE, "%s and %s must have the same shape", kn, vn);
  if (k->shape[0] != q->shape[0]) return fail(RA_E_SHAPE, "batch of q and %s differ", kn);
  if (k->shape[3] != q->shape[3]) return fail(RA_E_SHAPE, "head_dim of q and %s differ", kn);
  if (k->shape[2] < 1 || q->shape[2] < 1) return fail(RA_E_SHAPE, "head counts must be >= 1");
  if (q->shape[2] % k->shape[2] != 0)
    return fail(RA_E_SHAPE, "query heads (%lld) must be a multiple of kv heads (%lld)", (long long)q->shape[2],
                (long long)k->shape[2]);
  const int64_t d = q->shape[3];
  if (d != 64 && d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  const int64_t lim = std::numeric_limits<int32_t>::max();
  if (q->shape[0] > lim || q->shape[1] > lim || q->shape[2] > lim)
    return fail(RA_E_RANGE, "q dimensions exceed 2^31 - 1");
  // the kernels walk a block's keys with 32-bit counters
  if (k->shape[1] > (int64_t(1) << 29)) return fail(RA_E_RANGE, "%s/%s hold more than 2^29 keys per block", kn, vn);
  // the tile loads address the rows of one key tile with 32-bit byte offsets
  if (k->stride[1] > (int64_t(1) << 24) || v->stride[1] > (int64_t(1) << 24))
    return fail(RA_E_RANGE, "%s/%s sequence stride exceeds 2^24 elements", kn, vn);
  return RA_OK;
}

// A launch of ceil(rows / bm) * heads * B workgroups of `threads` threads: HIP
// takes at most 2^32 - 1 work-items along the grid's x dimension.
int check_grid(int64_t rows, int64_t bm, int64_t heads, int64_t B, int64_t threads) {
  const int64_t wg = ((rows + bm - 1) / bm) * heads * B;
  if (wg > (int64_t)std::numeric_limits<uint32_t>::max() / threads)
    return fail(RA_E_RANGE, "launch too large: %lld workgroups of %lld threads exceed 2^32 - 1 work-items",
                (long long)wg, (long long)threads);
  return RA_OK;
}

void set_bshd(const ra_tensor* t, int64_t& sb, int64_t& ss, int64_t& sh) {
  sb = t->stride[0];
  ss = t->stride[1];
  sh = t->stride[2];
}

void set_rows(const ra_tensor* t, int64_t& sb, int64_t& sh, int64_t& ss) {
  sb = t->stride[0];
  sh = t->stride[1];
  ss = t->stride[2];
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// A state kernel (init, merge, finalize) over [B, S, H, d] rows.
int check_state_grid(int64_t B, int64_t H, int64_t S, int64_t d) {
  if (B > std::numeric_limits<int32_t>::max() || H > std::numeric_limits<int32_t>::max() ||
      S > std::numeric_limits<int32_t>::max())
    return fail(RA_E_RANGE, "state dimensions exceed 2^31 - 1");
  const int64_t wg = ra_state_workgroups(B, H, S, d);
  if (wg > (int64_t)std::numeric_limits<uint32_t>::max() / RA_STATE_THREADS)
    return fail(RA_E_RANGE, "launch too large: %lld workgroups of %d threads exceed 2^32 - 1 work-items",
                (long long)wg, RA_STATE_THREADS);
  return RA_OK;
}

int check_out(const ra_tensor* o, const ra_tensor* like, const char* name) {
  int e = check_bshd(o, name);
  if (e) return e;
  if (!same_shape(o, like)) return fail(RA_E_SHAPE, "%s must have the shape of %s", name, "the queries");
  return RA_OK;
}

// ---- the allocation-free backward's workspace
//
// ra_rank_share_bwd_noalloc keeps D_i = <dO_i, O_i> (the `delta` workspace of
// ra_rank_share_bwd) in this array instead of a caller buffer.  In host code
// the name is a host-side stand-in, never a device address: each device holds
// its own copy, whose address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch_ptr.
// The prep kernel writes every entry a call reads, so nothing needs clearing;
// calls that overlap on one device share the array and race.
constexpr int64_t kNoallocMaxRows = int64_t(1) << 20;  // 4 MiB of fp32 per device
static __device__ __align__(256) float scratch[kNoallocMaxRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use).
int scratch_of_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_E_RANGE, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RA_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

int ra_state_init(const ra_tensor* o_acc, const ra_tensor* m, const ra_tensor* l, const ra_opts* opts) {
  int e = check_bshd(o_acc, "o_acc");
  if (e) return e;
  if (o_acc->dtype != RA_F32) return fail(RA_E_DTYPE, "o_acc must be fp32");
  const int64_t B = o_acc->shape[0], S = o_acc->shape[1], H = o_acc->shape[2], d = o_acc->shape[3];
  if ((e = check_rows(m, "m", B, H, S)) || (e = check_rows(l, "l", B, H, S))) return e;
  if (d != 64 && d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  if ((e = check_state_grid(B, H, S, d))) return e;
  if (B * S * H == 0) return ok();
  RaInitArgs a{};
  a.oacc = (float*)o_acc->data;
  set_bshd(o_acc, a.oa_sb, a.oa_ss, a.oa_sh);
  a.m = (float*)m->data;
  set_rows(m, a.m_sb, a.m_sh, a.m_ss);
  a.l = (float*)l->data;
  set_rows(l, a.l_sb, a.l_sh, a.l_ss);
  a.B = (int32_t)B; a.H = (int32_t)H; a.S = (int32_t)S; a.d = (int32_t)d;
  return launched(ra_launch_init(a, stream_of(opts)), "ra_state_init launch");
}

int ra_step(const ra_tensor* q, const ra_tensor* k_blk, const ra_tensor* v_blk, const ra_tensor* o_acc,
            const ra_tensor* m, const ra_tensor* l, int64_t q_off, int64_t kv_off, int causal,
            const ra_opts* opts) {
  int e = check_qkv(q, k_blk, v_blk, "k_blk", "v_blk");
  if (e) return e;
  const int64_t B = q->shape[0], nq = q->shape[1], hq = q->shape[2], d = q->shape[3];
  const int64_t nkv = k_blk->shape[1];
  if ((e = check_bshd(o_acc, "o_acc"))) return e;
  if (o_acc->dtype != RA_F32) return fail(RA_E_DTYPE, "o_acc must be fp32");
  if (!same_shape(o_acc, q)) return fail(RA_E_SHAPE, "o_acc must have the shape of q");
  if ((e = check_rows(m, "m", B, hq, nq)) || (e = check_rows(l, "l", B, hq, nq))) return e;
  if (q_off < 0 || kv_off < 0) return fail(RA_E_RANGE, "q_off and kv_off must be >= 0");
  const int64_t bm = q->dtype == RA_BF16 ? RA_BF16_BM : RA_F32_BM;
  if ((e = check_grid(nq, bm, hq, B, q->dtype == RA_BF16 ? RA_BF16_THREADS : RA_F32_THREADS))) return e;
  if (B == 0 || nq == 0 || ra_plan_class(q_off, nq, kv_off, nkv, causal) == RA_CLASS_SKIP) return ok();

  RaAttnArgs a{};
  a.nsplit = 1;
  a.kv_end = kv_off + nkv;
  a.q = q->data; set_bshd(q, a.q_sb, a.q_ss, a.q_sh);
  a.k = k_blk->data; set_bshd(k_blk, a.k_sb, a.k_ss, a.k_sh);
  a.v = v_blk->data; set_bshd(v_blk, a.v_sb, a.v_ss, a.v_sh);
  a.B = (int32_t)B; a.Hq = (int32_t)hq; a.Hkv = (int32_t)k_blk->shape[2]; a.nq = (int32_t)nq;
  a.nkv = nkv; a.q_off = q_off; a.kv_off = kv_off;
  a.ring = 0; a.P = 1; a.rank = 0; a.causal = causal ? 1 : 0;
  a.c = resolve_scale(opts, d) * 1.4426950408889634f;
  a.state_in = 1; a.out_state = 1;
  a.oacc = (float*)o_acc->data; set_bshd(o_acc, a.oa_sb, a.oa_ss, a.oa_sh);
  a.m = (float*)m->data; set_rows(m, a.m_sb, a.m_sh, a.m_ss);
  a.l = (float*)l->data; set_rows(l, a.l_sb, a.l_sh, a.l_ss);
  hipStream_t st = stream_of(opts);
  return launched(q->dtype == RA_BF16 ? ra_launch_attn_bf16(a, (int)d, st) : ra_launch_attn_f32(a, (int)d, st),
                  "ra_step launch");
}

int ra_finalize(const ra_tensor* o_acc, const ra_tensor* l, const ra_opts* opts) {
  int e = check_bshd(o_acc, "o_acc");
  if (e) return e;
  if (o_acc->dtype != RA_F32) return fail(RA_E_DTYPE, "o_acc must be fp32");
  const int64_t B = o_acc->shape[0], S = o_acc->shape[1], H = o_acc->shape[2], d = o_acc->shape[3];
  if ((e = check_rows(l, "l", B, H, S))) return e;
  if (d != 64 && d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  const ra_tensor* o_out = opts ? opts->o_out : nullptr;
  const ra_tensor* lse = opts ? opts->lse_out : nullptr;
  const ra_tensor* mt = opts ? opts->m : nullptr;
  if (o_out && (e = check_out(o_out, o_acc, "o_out"))) return e;
  if (lse) {
    if (!mt) return fail(RA_E_NULL, "lse_out needs opts->m");
    if ((e = check_rows(mt, "m", B, H, S)) || (e = check_rows(lse, "lse_out", B, H, S))) return e;
  }
  if ((e = check_state_grid(B, H, S, d))) return e;
  if (B * S * H == 0) return ok();
  RaFinArgs a{};
  a.oacc = (const float*)o_acc->data; set_bshd(o_acc, a.oa_sb, a.oa_ss, a.oa_sh);
  a.l = (const float*)l->data; set_rows(l, a.l_sb, a.l_sh, a.l_ss);
  if (o_out) {
    a.o = o_out->data; set_bshd(o_out, a.o_sb, a.o_ss, a.o_sh); a.o_bf16 = o_out->dtype == RA_BF16;
  } else {
    a.o = o_acc->data; set_bshd(o_acc, a.o_sb, a.o_ss, a.o_sh); a.o_bf16 = 0;
  }
  if (lse) {
    a.m = (const float*)mt->data; set_rows(mt, a.m_sb, a.m_sh, a.m_ss);
    a.lse = (float*)lse->data; set_rows(lse, a.lse_sb, a.lse_sh, a.lse_ss);
  }
  a.B = (int32_t)B; a.S = (int32_t)S; a.H = (int32_t)H; a.d = (int32_t)d;
  return launched(ra_launch_finalize(a, stream_of(opts)), "ra_finalize launch");
}

int ra_merge(const ra_tensor* o_acc, const ra_tensor* m, const ra_tensor* l, const ra_tensor* o_b,
             const ra_tensor* m_b, const ra_tensor* l_b, const ra_opts* opts) {
  int e;
  if ((e = check_bshd(o_acc, "o_acc")) || (e = check_bshd(o_b, "o_b"))) return e;
  if (o_acc->dtype != RA_F32 || o_b->dtype != RA_F32) return fail(RA_E_DTYPE, "o_acc and o_b must be fp32");
  if (!same_shape(o_acc, o_b)) return fail(RA_E_SHAPE, "o_b must have the shape of o_acc");
  const int64_t B = o_acc->shape[0], S = o_acc->shape[1], H = o_acc->shape[2], d = o_acc->shape[3];
  if ((e = check_rows(m, "m", B, H, S)) || (e = check_rows(l, "l", B, H, S)) || (e = check_rows(m_b, "m_b", B, H, S)) ||
      (e = check_rows(l_b, "l_b", B, H, S)))
    return e;
  if (d != 64 && d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  if ((e = check_state_grid(B, H, S, d))) return e;
  if (B * S * H == 0) return ok();
  RaMergeArgs a{};
  a.oa = (float*)o_acc->data; set_bshd(o_acc, a.oa_sb, a.oa_ss, a.oa_sh);
  a.ma = (float*)m->data; set_rows(m, a.ma_sb, a.ma_sh, a.ma_ss);
  a.la = (float*)l->data; set_rows(l, a.la_sb, a.la_sh, a.la_ss);
  a.ob = (const float*)o_b->data; set_bshd(o_b, a.ob_sb, a.ob_ss, a.ob_sh);
  a.mb = (const float*)m_b->data; set_rows(m_b, a.mb_sb, a.mb_sh, a.mb_ss);
  a.lb = (const float*)l_b->data; set_rows(l_b, a.lb_sb, a.lb_sh, a.lb_ss);
  a.B = (int32_t)B; a.H = (int32_t)H; a.S = (int32_t)S; a.d = (int32_t)d;
  return launched(ra_launch_merge(a, stream_of(opts)), "ra_merge launch");
}

// One rank's share in one launch.  zigzag == 0: the local rows are block
// `rank` of P contiguous blocks; zigzag == 1: they are chunks rank and
// 2P-1-rank of 2P chunks (the load-balanced share), each chunk folding all 2P
// key chunks in its own ring order.
static int rank_share(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, int P, int rank, int causal,
                      const ra_opts* opts, int zigzag, int64_t n_valid) {
  const char* fn = zigzag ? "ra_rank_share_zigzag" : (n_valid >= 0 ? "ra_rank_share_padded" : "ra_rank_share");
  int e = check_qkv(q, k, v, "k", "v");
  if (e) return e;
  if (!opts || !opts->o_out) return fail(RA_E_NULL, "%s needs opts->o_out", fn);
  if (P < 1) return fail(RA_E_RANGE, "P must be >= 1 (got %d)", P);
  if (rank < 0 || rank >= P) return fail(RA_E_RANGE, "rank %d outside [0, %d)", rank, P);
  const int64_t B = q->shape[0], nq = q->shape[1], hq = q->shape[2], d = q->shape[3];
  const int64_t N = k->shape[1];
  const int64_t parts = zigzag ? 2 * (int64_t)P : P;
  if (N % parts != 0)
    return fail(RA_E_SHAPE, "sequence length %lld is not divisible by %s = %lld (no implicit padding)",
                (long long)N, zigzag ? "2P" : "P", (long long)parts);
  if (n_valid > N) return fail(RA_E_RANGE, "n_valid %lld exceeds the padded length %lld", (long long)n_valid, (long long)N);
  if (n_valid == 0 && N > 0) return fail(RA_E_RANGE, "n_valid must be >= 1");
  const int64_t nb = N / parts;  // block (contiguous) or chunk (zigzag) length
  const int64_t rows = zigzag ? 2 * nb : nb;
  if (nq != rows)
    return fail(RA_E_SHAPE, "local query block has %lld rows, expected %s = %lld", (long long)nq,
                zigzag ? "2 N/(2P)" : "N/P", (long long)rows);
  if ((e = check_out(opts->o_out, q, "o_out"))) return e;
  if (opts->lse_out && (e = check_rows(opts->lse_out, "lse_out", B, hq, nq))) return e;
  const int64_t bm = q->dtype == RA_BF16 ? RA_BF16_BM : RA_F32_BM;
  if ((e = check_grid(zigzag ? 2 * ((nb + bm - 1) / bm) * bm : nq, bm, hq, B,
                      q->dtype == RA_BF16 ? RA_BF16_THREADS : RA_F32_THREADS)))
    return e;
  if (B == 0 || nq == 0) return ok();

  RaAttnArgs a{};
  a.q = q->data; set_bshd(q, a.q_sb, a.q_ss, a.q_sh);
  a.k = k->data; set_bshd(k, a.k_sb, a.k_ss, a.k_sh);
  a.v = v->data; set_bshd(v, a.v_sb, a.v_ss, a.v_sh);
  a.B = (int32_t)B; a.Hq = (int32_t)hq; a.Hkv = (int32_t)k->shape[2]; a.nq = (int32_t)nq;
  a.nkv = nb; a.q_off = (int64_t)rank * nb; a.kv_off = 0;
  a.ring = 1; a.P = (int32_t)parts; a.rank = rank; a.causal = causal ? 1 : 0;
  a.nsplit = 1;
  a.kv_end = n_valid >= 0 ? n_valid : N;
  if (zigzag) {
    a.nsplit = 2; a.qc = nb;
    a.rank2 = (int32_t)(parts - 1 - rank); a.q_off2 = (parts - 1 - rank) * nb;
  }
  a.c = resolve_scale(opts, d) * 1.4426950408889634f;
  a.state_in = 0; a.out_state = 0;
  a.o = opts->o_out->data; set_bshd(opts->o_out, a.o_sb, a.o_ss, a.o_sh); a.o_bf16 = opts->o_out->dtype == RA_BF16;
  if (opts->lse_out) { a.lse = (float*)opts->lse_out->data; set_rows(opts->lse_out, a.lse_sb, a.lse_sh, a.lse_ss); }
  hipStream_t st = stream_of(opts);
  return launched(q->dtype == RA_BF16 ? ra_launch_attn_bf16(a, (int)d, st) : ra_launch_attn_f32(a, (int)d, st),
                  zigzag ? "ra_rank_share_zigzag launch" : "ra_rank_share launch");
}

int ra_rank_share(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, int P, int rank, int causal,
                  const ra_opts* opts) {
  return rank_share(q, k, v, P, rank, causal, opts, 0, -1);
}

int ra_rank_share_padded(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, int P, int rank, int causal,
                         int64_t n_valid, const ra_opts* opts) {
  if (n_valid < 0) return fail(RA_E_RANGE, "n_valid must be >= 1");
  return rank_share(q, k, v, P, rank, causal, opts, 0, n_valid);
}

int ra_rank_share_zigzag(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, int P, int rank, int causal,
                         const ra_opts* opts) {
  return rank_share(q, k, v, P, rank, causal, opts, 1, -1);
}

static int rank_share_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* o,
                          const ra_tensor* lse, const ra_tensor* dout, int P, int rank, int causal,
                          const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv, const ra_tensor* delta,
                          const ra_opts* opts, int zigzag, int64_t n_valid, bool noalloc = false) {
  const char* fn = noalloc ? "ra_rank_share_bwd_noalloc"
                           : (zigzag ? "ra_rank_share_zigzag_bwd"
                                     : (n_valid >= 0 ? "ra_rank_share_padded_bwd" : "ra_rank_share_bwd"));
  int e = check_qkv(q, k, v, "k", "v");
  if (e) return e;
  if (q->dtype != RA_BF16) return fail(RA_E_UNSUPPORTED, "%s takes bf16 q, k, v", fn);
  if (P < 1) return fail(RA_E_RANGE, "P must be >= 1 (got %d)", P);
  if (rank < 0 || rank >= P) return fail(RA_E_RANGE, "rank %d outside [0, %d)", rank, P);
  const int64_t B = q->shape[0], nq = q->shape[1], hq = q->shape[2], d = q->shape[3];
  const int64_t N = k->shape[1];
  const int64_t parts = zigzag ? 2 * (int64_t)P : P;
  if (N % parts != 0)
    return fail(RA_E_SHAPE, "sequence length %lld is not divisible by %s = %lld (no implicit padding)",
                (long long)N, zigzag ? "2P" : "P", (long long)parts);
  if (n_valid > N) return fail(RA_E_RANGE, "n_valid %lld exceeds the padded length %lld", (long long)n_valid, (long long)N);
  if (n_valid == 0 && N > 0) return fail(RA_E_RANGE, "n_valid must be >= 1");
  const int64_t nb = N / P;  // local rows either way (zigzag: two chunks of N/(2P))
  if (nq != nb) return fail(RA_E_SHAPE, "local query block has %lld rows, expected N/P = %lld", (long long)nq, (long long)nb);
  if ((e = check_out(o, q, "o")) || (e = check_out(dout, q, "dout")) || (e = check_out(dq, q, "dq"))) return e;
  if (o->dtype != RA_BF16 || dout->dtype != RA_BF16) return fail(RA_E_DTYPE, "o and dout must be bf16");
  // the dK/dV kernel loads q and dout tiles with 32-bit byte offsets, like k and v
  if (q->stride[1] > (int64_t(1) << 24) || dout->stride[1] > (int64_t(1) << 24))
    return fail(RA_E_RANGE, "q/dout sequence stride exceeds 2^24 elements");
  if (dq->dtype != RA_F32) return fail(RA_E_DTYPE, "dq must be fp32");
  if ((e = check_bshd(dk, "dk")) || (e = check_bshd(dv, "dv"))) return e;
  if (!same_shape(dk, k) || !same_shape(dv, k)) return fail(RA_E_SHAPE, "dk and dv must have the shape of k");
  if (dk->dtype != RA_F32 || dv->dtype != RA_F32) return fail(RA_E_DTYPE, "dk and dv must be fp32");
  if ((e = check_rows(lse, "lse", B, hq, nq))) return e;
  if (noalloc) {
    if (B * hq * nq > kNoallocMaxRows)
      return fail(RA_E_RANGE, "%s: B * Hq * Nq = %lld query rows exceed its workspace of %lld rows", fn,
                  (long long)(B * hq * nq), (long long)kNoallocMaxRows);
  } else if ((e = check_rows(delta, "delta", B, hq, nq))) {
    return e;
  }
  const int64_t qrows = zigzag ? 2 * ((N / parts + RA_BWD_BM - 1) / RA_BWD_BM) * RA_BWD_BM : nq;
  if ((e = check_grid(qrows, RA_BWD_BM, hq, B, RA_BWD_THREADS)) ||
      (e = check_grid(N, RA_BWD_BM, k->shape[2], B, RA_BWD_THREADS)) ||
      (e = check_grid(nq, RA_BWD_THREADS, hq, B, RA_BWD_THREADS)))  // prep: one thread per query row
    return e;
  if (B == 0 || nq == 0) return ok();
  float* ws = nullptr;
  if (noalloc && (e = scratch_of_current_device(&ws))) return e;

  RaBwdArgs a{};
  a.q = q->data; set_bshd(q, a.q_sb, a.q_ss, a.q_sh);
  a.k = k->data; set_bshd(k, a.k_sb, a.k_ss, a.k_sh);
  a.v = v->data; set_bshd(v, a.v_sb, a.v_ss, a.v_sh);
  a.o = o->data; set_bshd(o, a.o_sb, a.o_ss, a.o_sh);
  a.dout = dout->data; set_bshd(dout, a.do_sb, a.do_ss, a.do_sh);
  a.lse = (const float*)lse->data; set_rows(lse, a.lse_sb, a.lse_sh, a.lse_ss);
  if (noalloc) {  // [B, Hq, Nq], contiguous
    a.delta = ws; a.de_sb = hq * nq; a.de_sh = nq; a.de_ss = 1;
  } else {
    a.delta = (float*)delta->data; set_rows(delta, a.de_sb, a.de_sh, a.de_ss);
  }
  a.dq = (float*)dq->data; set_bshd(dq, a.dq_sb, a.dq_ss, a.dq_sh);
  a.dk = (float*)dk->data; set_bshd(dk, a.dk_sb, a.dk_ss, a.dk_sh);
  a.dv = (float*)dv->data; set_bshd(dv, a.dv_sb, a.dv_ss, a.dv_sh);
  a.B = (int32_t)B; a.Hq = (int32_t)hq; a.Hkv = (int32_t)k->shape[2]; a.nq = (int32_t)nq;
  a.N = N; a.nb = nb; a.q_off = (int64_t)rank * nb;
  a.P = P; a.rank = rank; a.causal = causal ? 1 : 0;
  a.nsplit = 1;
  a.kv_end = n_valid >= 0 ? n_valid : N;
  if (zigzag) {
    const int64_t c = N / parts;
    a.nsplit = 2; a.qc = c; a.q_off = (int64_t)rank * c;
    a.rank2 = (int32_t)(parts - 1 - rank); a.q_off2 = (parts - 1 - rank) * c;
  }
  a.scale = resolve_scale(opts, d);
  a.c = a.scale * 1.4426950408889634f;
  return launched(ra_launch_bwd(a, (int)d, stream_of(opts)), fn);
}

int ra_rank_share_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* o,
                      const ra_tensor* lse, const ra_tensor* dout, int P, int rank, int causal, const ra_tensor* dq,
                      const ra_tensor* dk, const ra_tensor* dv, const ra_tensor* delta, const ra_opts* opts) {
  return rank_share_bwd(q, k, v, o, lse, dout, P, rank, causal, dq, dk, dv, delta, opts, 0, -1);
}

int ra_rank_share_bwd_noalloc(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* o,
                              const ra_tensor* lse, const ra_tensor* dout, int P, int rank, int causal,
                              const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv, const ra_opts* opts) {
  return rank_share_bwd(q, k, v, o, lse, dout, P, rank, causal, dq, dk, dv, nullptr, opts, 0, -1, true);
}

int ra_rank_share_padded_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* o,
                             const ra_tensor* lse, const ra_tensor* dout, int P, int rank, int causal,
                             int64_t n_valid, const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv,
                             const ra_tensor* delta, const ra_opts* opts) {
  if (n_valid < 0) return fail(RA_E_RANGE, "n_valid must be >= 1");
  return rank_share_bwd(q, k, v, o, lse, dout, P, rank, causal, dq, dk, dv, delta, opts, 0, n_valid);
}

int ra_rank_share_zigzag_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* o,
                             const ra_tensor* lse, const ra_tensor* dout, int P, int rank, int causal,
                             const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv, const ra_tensor* delta,
                             const ra_opts* opts) {
  return rank_share_bwd(q, k, v, o, lse, dout, P, rank, causal, dq, dk, dv, delta, opts, 1, -1);
}

int64_t ra_ring_block(int64_t P, int64_t rank, int64_t s) {
  if (P < 1) return -1;
  return ra_plan_ring_block(P, rank, s);
}

int ra_classify(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal) {
  return ra_plan_class(q_off, nq, kv_off, nkv, causal);
}

int64_t ra_plan_tiles(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal, int64_t bm, int64_t bn,
                      int8_t* out, int64_t out_len) {
  if (bm < 1 || bn < 1 || nq < 0 || nkv < 0) return fail(RA_E_RANGE, "tile sizes must be >= 1, lengths >= 0");
  const int64_t ti = (nq + bm - 1) / bm, tj = (nkv + bn - 1) / bn;
  if (ti * tj > out_len) return fail(RA_E_RANGE, "out holds %lld entries, %lld needed", (long long)out_len, (long long)(ti * tj));
  if (ti * tj > 0 && !out) return fail(RA_E_NULL, "out is NULL");
  for (int64_t i = 0; i < ti; ++i)
    for (int64_t j = 0; j < tj; ++j) {
      const int64_t rq = (i + 1) * bm <= nq ? bm : nq - i * bm;
      const int64_t rk = (j + 1) * bn <= nkv ? bn : nkv - j * bn;
      out[i * tj + j] = (int8_t)ra_plan_class(q_off + i * bm, rq, kv_off + j * bn, rk, causal);
    }
  return ti * tj;
}

int ra_tile_shape(int32_t dtype, int64_t d, int64_t* bm, int64_t* bn) {
  if (!bm || !bn) return fail(RA_E_NULL, "bm and bn must not be NULL");
  if (!dtype_valid(dtype)) return fail(RA_E_DTYPE, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported", (long long)d);
  *bm = dtype == RA_BF16 ? RA_BF16_BM : RA_F32_BM;
  *bn = dtype == RA_BF16 ? RA_BF16_BN : RA_F32_BN;
  return ok();
}

double ra_flops(int64_t nq, int64_t nkv, int64_t q_off, int64_t kv_off, int64_t hq, int64_t d, int causal) {
  if (nq < 0 || nkv < 0 || q_off < 0 || kv_off < 0 || hq < 0 || d < 0) return -1.0;
  const int c = ra_plan_class(q_off, nq, kv_off, nkv, causal);
  const double unit = 4.0 * (double)nq * (double)nkv * (double)d * (double)hq;
  return c == RA_CLASS_FULL ? unit : (c == RA_CLASS_PARTIAL ? 0.5 * unit : 0.0);
}

double ra_share_flops(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal) {
  if (P < 1 || N % P != 0 || rank < 0 || rank >= P) return -1.0;
  const int64_t nb = N / P;
  double f = 0.0;
  const double unit = 4.0 * (double)d * (double)hq * (double)nb * (double)nb * (double)B;
  for (int64_t s = 0; s < P; ++s) {
    const int c = ra_plan_class(rank * nb, nb, ra_plan_ring_block(P, rank, s) * nb, nb, causal);
    f += c == RA_CLASS_FULL ? unit : (c == RA_CLASS_PARTIAL ? 0.5 * unit : 0.0);
  }
  return f;
}

double ra_share_flops_zigzag(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal) {
  if (P < 1 || N % (2 * P) != 0 || rank < 0 || rank >= P) return -1.0;
  const int64_t c = N / (2 * P), chunks = 2 * P;
  const double unit = 4.0 * (double)d * (double)hq * (double)c * (double)c * (double)B;
  double f = 0.0;
  for (const int64_t qa : {(int64_t)rank, chunks - 1 - rank})
    for (int64_t t = 0; t < chunks; ++t) {
      const int cl = ra_plan_class(qa * c, c, t * c, c, causal);
      f += cl == RA_CLASS_FULL ? unit : (cl == RA_CLASS_PARTIAL ? 0.5 * unit : 0.0);
    }
  return f;
}

const char* ra_last_error(void) { return g_err; }

const char* ra_version(void) { return "libringattn 0.1.0 (gfx950)"; }

}  // extern "C"
