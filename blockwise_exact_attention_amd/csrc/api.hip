// C ABI of the attention library: argument checks, mask-bound folding and
// dispatch.  Every check runs before the first HIP call, so a rejected call
// launches nothing and touches no device state.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "launch.hpp"

namespace {

using bea::AttnShape;
static_assert(ATTN_RING_MAX_CHUNKS == bea::kMaxChunks, "chunk limit of the one-launch share");

// a, b: counts that may be zero (batch, sequence length); c, d: layout
// sizes that must be positive (heads, head dim).
bool sizes_ok(long long a, long long b, long long c, long long d) {
  if (a < 0 || b < 0 || c <= 0 || d <= 0) return false;
  if (a == 0 || b == 0) return true;
  // every element count (and its byte size) must stay far below 2^62
  const long long lim = 1LL << 58;
  if (a > lim / b) return false;
  const long long ab = a * b;
  if (ab > lim / c) return false;
  const long long abc = ab * c;
  return abc <= lim / d;
}

// A pointer may be NULL only where its tensor has no elements.
bool missing(const void* p, long long bytes) { return p == nullptr && bytes > 0; }

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, long long bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int32_t sat32(long long x) {
  if (x < INT_MIN) return INT_MIN;
  if (x > INT_MAX) return INT_MAX;
  return (int32_t)x;
}

// Fold causal, the window and the offsets into bounds on j - i:
// key j is allowed for row i iff dlo <= j - i <= dhi.  With
// delta = q_offset - k_offset: causal kpos <= qpos is j - i <= delta, the
// window qpos - win_l <= kpos <= qpos + win_r is
// delta - win_l <= j - i <= delta + win_r.  |delta| is clamped to 2^40 first:
// |j - i| < 2^31, so larger values give the same answer, and the sums below
// cannot overflow.  Saturating to int32 keeps every comparison exact.
void mask_bounds(int causal, int win_l, int win_r, long long q_offset,
                 long long k_offset, int* dlo, int* dhi) {
  const long long cap = 1LL << 40;
  long long qo = q_offset, ko = k_offset;
  // q_offset - k_offset without overflow, clamped
  long long delta;
  if (qo >= 0 && ko < 0 && qo > LLONG_MAX + ko) delta = cap;
  else if (qo < 0 && ko > 0 && qo < LLONG_MIN + ko) delta = -cap;
  else delta = qo - ko;
  if (delta > cap) delta = cap;
  if (delta < -cap) delta = -cap;
  long long lo = LLONG_MIN / 2, hi = LLONG_MAX / 2;
  if (causal) hi = delta;
  if (win_r >= 0 && delta + win_r < hi) hi = delta + win_r;
  if (win_l >= 0) lo = delta - win_l;
  *dlo = sat32(lo);
  *dhi = sat32(hi);
}

int check_attn_args(int n, int l_q, int l_k, int h, int h_kv, int d,
                    float scale, int dtype) {
  if (!sizes_ok(n, l_q, h, d) || !sizes_ok(n, l_k, h_kv, d))
    return ATTN_ERR_SHAPE;
  if (h % h_kv != 0) return ATTN_ERR_SHAPE;
  // grid sizes (q tiles x heads; split key tiles x key/value heads) must fit
  // a 32-bit launch
  if ((long long)((l_q + 63) / 64) * n * h > INT_MAX) return ATTN_ERR_SHAPE;
  if ((long long)((l_k + 63) / 64) * n * h_kv * 4 > INT_MAX) return ATTN_ERR_SHAPE;
  // the attention kernels launch up to four work-items per query row and
  // per key row, and a launch counts its work-items in 32 bits (the row
  // passes and elementwise kernels walk capped grids instead)
  if ((long long)n * l_q * h * 4 > (long long)UINT_MAX) return ATTN_ERR_SHAPE;
  if ((long long)n * l_k * h_kv * 4 > (long long)UINT_MAX) return ATTN_ERR_SHAPE;
  // the kernels address a 64-row tile with 32-bit offsets from its first
  // row: a row (h or h_kv heads of d float32 values at most) must stay
  // below 32 MiB
  if ((long long)h * d * 4 > (1LL << 25)) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int n, int l_q, int l_k, int h, int h_kv, int d, float scale,
             int causal, int win_l, int win_r, long long q_offset,
             long long k_offset, void* stream, int dtype) {
  int st = check_attn_args(n, l_q, l_k, h, h_kv, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const long long es = dtype == ATTN_BF16 ? 2 : 4;
  const long long qb = (long long)n * l_q * h * d * es;
  const long long kb = (long long)n * l_k * h_kv * d * es;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(q, qb) || missing(k, kb) || missing(v, kb) || missing(out, qb) ||
      missing(lse, lb))
    return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(out, 16) || !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  const Range rq = range(q, qb), rk = range(k, kb), rv = range(v, kb),
              ro = range(out, qb), rl = range(lse, lb);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) ||
      overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ro))
    return ATTN_ERR_ALIAS;
  if (qb == 0) return ATTN_OK;  // no query rows: nothing to write

  (void)hipGetLastError();  // clear a stale error so the check below is ours
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // no keys: every row is empty, O = 0 and LSE = -inf (O cleared as 32-bit
  // words: d * es is a multiple of 4)
  if (kb == 0)
    return finish(bea::launch_acc_init(static_cast<float*>(out), lse, n, l_q, h,
                                       (int)(d * es / 4), hs));
  AttnShape s{n, l_q, l_k, h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
  mask_bounds(causal, win_l, win_r, q_offset, k_offset, &s.dlo, &s.dhi);
  if (dtype == ATTN_F32) return finish(bea::launch_fwd_f32(q, k, v, out, lse, s, hs));
  const bea::FwdChunk ch{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), l_k,
                         s.dlo, s.dhi};
  if (bea::fwd_pipe_preferred(&ch, 1, s))
    return finish(bea::launch_fwd_pipe(q, &ch, 1, out, lse, s, hs));
  return finish(bea::launch_fwd_bf16(q, k, v, out, lse, s, hs));
}

int attn_fwd_acc(const void* q, const void* k, const void* v, float* out_acc,
                 float* lse_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                 float scale, int causal, int win_l, int win_r,
                 long long q_offset, long long k_offset, void* stream, int dtype) {
  int st = check_attn_args(n, l_q, l_k, h, h_kv, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const long long es = dtype == ATTN_F32 ? 4 : 2;
  const long long qb = (long long)n * l_q * h * d * es;
  const long long kb = (long long)n * l_k * h_kv * d * es;
  const long long ab = (long long)n * l_q * h * d * 4;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(q, qb) || missing(k, kb) || missing(v, kb) || missing(out_acc, ab) ||
      missing(lse_acc, lb))
    return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(out_acc, 16) || !aligned(lse_acc, 4))
    return ATTN_ERR_ALIGN;
  const Range rq = range(q, qb), rk = range(k, kb), rv = range(v, kb),
              ra = range(out_acc, ab), rl = range(lse_acc, lb);
  if (overlap(ra, rq) || overlap(ra, rk) || overlap(ra, rv) ||
      overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ra))
    return ATTN_ERR_ALIAS;
  if (qb == 0) return ATTN_OK;  // no query rows: nothing to merge
  (void)hipGetLastError();
  // an empty chunk: every block row is (0, -inf), so rows with a result keep
  // it and rows still at -inf become O = 0
  if (kb == 0)
    return finish(bea::launch_acc_clear_empty(out_acc, lse_acc, n, l_q, h, d,
                                              static_cast<hipStream_t>(stream)));

  AttnShape s{n, l_q, l_k, h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
  mask_bounds(causal, win_l, win_r, q_offset, k_offset, &s.dlo, &s.dhi);
  const bea::FwdChunk ch{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), l_k,
                         s.dlo, s.dhi};
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_F32)
    return finish(bea::launch_fwd_f32(q, k, v, nullptr, nullptr, s, hs, out_acc, lse_acc));
  if (bea::fwd_pipe_preferred(&ch, 1, s))
    return finish(bea::launch_fwd_pipe(q, &ch, 1, nullptr, nullptr, s, hs, out_acc, lse_acc));
  return finish(bea::launch_fwd_bf16(q, k, v, nullptr, nullptr, s, hs, out_acc, lse_acc));
}

const char* attn_fwd_kernel_name(int n, int l_q, int l_k, int h, int h_kv, int d, float scale,
                                 int causal, int win_l, int win_r, long long q_offset,
                                 long long k_offset, int dtype, int fused) {
  if (check_attn_args(n, l_q, l_k, h, h_kv, d, scale, dtype) != ATTN_OK) return nullptr;
  if ((long long)n * l_q == 0 || l_k == 0) return nullptr;  // no attention kernel runs
  AttnShape s{n, l_q, l_k, h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
  mask_bounds(causal, win_l, win_r, q_offset, k_offset, &s.dlo, &s.dhi);
  if (dtype == ATTN_F32) {
    static const char* const names[2][2] = {
        {"fwd_f32_kernel<64, false>", "fwd_f32_kernel<64, true>"},
        {"fwd_f32_kernel<128, false>", "fwd_f32_kernel<128, true>"}};
    return names[d == 128 ? 1 : 0][fused ? 1 : 0];
  }
  const bea::FwdChunk ch{nullptr, nullptr, l_k, s.dlo, s.dhi};
  if (bea::fwd_pipe_preferred(&ch, 1, s)) return bea::fwd_pipe_kernel_name(&ch, 1, s, fused);
  return bea::fwd_bf16_kernel_name(s, fused);
}

int attn_fwd_ring(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                  const int* l_k_chunks, const long long* k_offsets, int n_chunks, void* out,
                  float* lse, int n, int l_q, int h, int h_kv, int d, float scale, int causal,
                  int win_l, int win_r, long long q_offset, void* stream, int dtype) {
  if (n_chunks < 1 || n_chunks > ATTN_RING_MAX_CHUNKS) return ATTN_ERR_SHAPE;
  if (k_chunks == nullptr || v_chunks == nullptr || l_k_chunks == nullptr ||
      k_offsets == nullptr)
    return ATTN_ERR_NULL;
  for (int c = 0; c < n_chunks; ++c) {
    const int st = check_attn_args(n, l_q, l_k_chunks[c], h, h_kv, d, scale, dtype);
    if (st != ATTN_OK) return st;
  }
  const long long es = dtype == ATTN_F32 ? 4 : 2;
  const long long qb = (long long)n * l_q * h * d * es;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(q, qb) || missing(out, qb) || missing(lse, lb)) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  const Range rq = range(q, qb), ro = range(out, qb), rl = range(lse, lb);
  if (overlap(ro, rq) || overlap(rl, rq) || overlap(rl, ro)) return ATTN_ERR_ALIAS;
  for (int c = 0; c < n_chunks; ++c) {
    const long long kb = (long long)n * l_k_chunks[c] * h_kv * d * es;
    if (missing(k_chunks[c], kb) || missing(v_chunks[c], kb)) return ATTN_ERR_NULL;
    if (!aligned(k_chunks[c], 16) || !aligned(v_chunks[c], 16)) return ATTN_ERR_ALIGN;
    const Range rk = range(k_chunks[c], kb), rv = range(v_chunks[c], kb);
    if (overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rk) || overlap(rl, rv))
      return ATTN_ERR_ALIAS;
  }
  if (qb == 0) return ATTN_OK;  // no query rows: nothing to write

  (void)hipGetLastError();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_F32) {
    // float32: out and lse are the accumulator itself (O = 0, LSE = -inf),
    // into which one fused step per chunk with keys merges its block
    hipError_t e = bea::launch_acc_init(static_cast<float*>(out), lse, n, l_q, h, d, hs);
    for (int c = 0; c < n_chunks && e == hipSuccess; ++c) {
      if ((long long)n * l_k_chunks[c] == 0) continue;
      AttnShape sc{n, l_q, l_k_chunks[c], h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
      mask_bounds(causal, win_l, win_r, q_offset, k_offsets[c], &sc.dlo, &sc.dhi);
      e = bea::launch_fwd_f32(q, k_chunks[c], v_chunks[c], nullptr, nullptr, sc, hs,
                              static_cast<float*>(out), lse);
    }
    return finish(e);
  }
  // chunks without keys add nothing: drop them
  bea::FwdChunk ch[bea::kMaxChunks];
  int m = 0;
  AttnShape s{n, l_q, 0, h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
  for (int c = 0; c < n_chunks; ++c) {
    if ((long long)n * l_k_chunks[c] == 0) continue;
    int dlo, dhi;
    mask_bounds(causal, win_l, win_r, q_offset, k_offsets[c], &dlo, &dhi);
    ch[m++] = bea::FwdChunk{static_cast<const uint16_t*>(k_chunks[c]),
                            static_cast<const uint16_t*>(v_chunks[c]), l_k_chunks[c], dlo, dhi};
  }
  // no keys at all: every row is empty, O = 0 and LSE = -inf
  if (m == 0)
    return finish(bea::launch_acc_init(static_cast<float*>(out), lse, n, l_q, h, d / 2, hs));
  s.l_k = ch[0].l_k;
  s.dlo = ch[0].dlo;
  s.dhi = ch[0].dhi;
  return finish(bea::launch_fwd_pipe(q, ch, m, out, lse, s, hs));
}

int attn_merge(float* out_acc, float* lse_acc, const void* out_blk,
               const float* lse_blk, int n, int l, int h, int d, int blk_dtype,
               void* stream) {
  if (!sizes_ok(n, l, h, d)) return ATTN_ERR_SHAPE;
  if ((long long)n * l * h > INT_MAX) return ATTN_ERR_SHAPE;  // rows of the merge grid
  if (blk_dtype != ATTN_F32 && blk_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  const long long es = blk_dtype == ATTN_BF16 ? 2 : 4;
  const long long ne = (long long)n * l * h * d;
  const long long nr = (long long)n * l * h;
  if (missing(out_acc, ne) || missing(lse_acc, nr) || missing(out_blk, ne) ||
      missing(lse_blk, nr))
    return ATTN_ERR_NULL;
  if (!aligned(out_acc, 16) || !aligned(out_blk, 16) || !aligned(lse_acc, 4) ||
      !aligned(lse_blk, 4))
    return ATTN_ERR_ALIGN;
  const Range ra = range(out_acc, ne * 4), rla = range(lse_acc, nr * 4),
              rb = range(out_blk, ne * es), rlb = range(lse_blk, nr * 4);
  if (overlap(ra, rla) || overlap(ra, rb) || overlap(ra, rlb) ||
      overlap(rla, rb) || overlap(rla, rlb))
    return ATTN_ERR_ALIAS;
  if (nr == 0) return ATTN_OK;
  (void)hipGetLastError();
  return finish(bea::launch_merge(out_acc, lse_acc, out_blk, lse_blk, n, l, h,
                                  d, blk_dtype == ATTN_BF16,
                                  static_cast<hipStream_t>(stream)));
}

int attn_hbm_copy(const void* src, void* dst, long long bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > (1LL << 40)) return ATTN_ERR_SHAPE;
  if (missing(src, bytes) || missing(dst, bytes)) return ATTN_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return ATTN_ERR_ALIGN;
  if (overlap(range(src, bytes), range(dst, bytes))) return ATTN_ERR_ALIAS;
  if (bytes == 0) return ATTN_OK;
  (void)hipGetLastError();
  return finish(bea::launch_hbm_copy(src, dst, bytes / 16, static_cast<hipStream_t>(stream)));
}

int attn_acc_init(float* out_acc, float* lse_acc, int n, int l, int h, int d,
                  void* stream) {
  if (!sizes_ok(n, l, h, d)) return ATTN_ERR_SHAPE;
  const long long ne = (long long)n * l * h * d;
  const long long nr = (long long)n * l * h;
  if (missing(out_acc, ne)) return ATTN_ERR_NULL;  // lse_acc may be NULL: O only
  if (!aligned(out_acc, 4) || !aligned(lse_acc, 4)) return ATTN_ERR_ALIGN;
  if (lse_acc && overlap(range(out_acc, ne * 4), range(lse_acc, nr * 4)))
    return ATTN_ERR_ALIAS;
  if (ne == 0) return ATTN_OK;
  (void)hipGetLastError();
  return finish(bea::launch_acc_init(out_acc, lse_acc, n, l, h, d,
                                     static_cast<hipStream_t>(stream)));
}

int attn_acc_cast(const float* out_acc, void* out, int n, int l, int h, int d,
                  int dtype, void* stream) {
  if (!sizes_ok(n, l, h, d)) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  const long long ne = (long long)n * l * h * d;
  const long long es = dtype == ATTN_BF16 ? 2 : 4;
  if (missing(out_acc, ne) || missing(out, ne)) return ATTN_ERR_NULL;
  if (!aligned(out_acc, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (overlap(range(out_acc, ne * 4), range(out, ne * es))) return ATTN_ERR_ALIAS;
  if (ne == 0) return ATTN_OK;
  (void)hipGetLastError();
  return finish(bea::launch_acc_cast(out_acc, out, n, l, h, d,
                                     dtype == ATTN_BF16,
                                     static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int n, int l_q, int l_k, int h, int h_kv,
                                int d) {
  if (!sizes_ok(n, l_q, h, d) || !sizes_ok(n, l_k, h_kv, d)) return 0;
  if (h % h_kv != 0) return 0;
  if (n == 0 || l_q == 0 || l_k == 0) return 0;  // nothing is launched
  return bea::bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d);
}

}  // extern "C"

namespace {

// Workspace of attn_bwd_static: one copy per device, held from the first
// load of the library's code object on that device until the process ends.
// Host code never passes `scratch` itself to a kernel or a copy (on the
// host the name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = (size_t)ATTN_BWD_STATIC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The scratch address on the device `stream` belongs to (the current device
// for the null stream), looked up once per device with that device current.
int scratch_for_stream(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    return ATTN_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

// Shared by attn_bwd, attn_bwd_acc and attn_bwd_static: argument checks
// (gradient outputs of gb bytes per element), then the launch; acc selects
// the accumulating kernels (gradients added to fp32 dq, dk, dv);
// use_scratch takes the workspace from the device's static scratch instead
// of the caller (workspace and workspace_bytes are then ignored).
int bwd_entry(const void* dout, const void* q, const void* k, const void* v,
              const void* out, const float* lse, void* dq, void* dk, void* dv,
              int n, int l_q, int l_k, int h, int h_kv, int d, float scale,
              int causal, int win_l, int win_r, long long q_offset,
              long long k_offset, void* workspace, size_t workspace_bytes,
              void* stream, int dtype, bool acc, bool use_scratch = false,
              bool prepared = false) {
  int st = check_attn_args(n, l_q, l_k, h, h_kv, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const bool f32 = dtype == ATTN_F32;
  const long long es = f32 ? 4 : 2;    // input element bytes
  const long long gb = acc ? 4 : es;   // gradient element bytes
  const long long qe = (long long)n * l_q * h * d;
  const long long ke = (long long)n * l_k * h_kv * d;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(dout, qe) || missing(q, qe) || missing(k, ke) || missing(v, ke) ||
      missing(out, qe) || missing(lse, lb) || missing(dq, qe) || missing(dk, ke) ||
      missing(dv, ke))
    return ATTN_ERR_NULL;
  const bool empty = qe == 0 || ke == 0;
  const size_t need = empty ? 0 : bea::bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d);
  if (use_scratch) {
    if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;
    workspace = nullptr;   // set after the checks
  } else if (missing(workspace, (long long)need) || workspace_bytes < need) {
    return ATTN_ERR_WORKSPACE;
  }
  if (!aligned(dout, 16) || !aligned(q, 16) || !aligned(k, 16) ||
      !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(workspace, 16))
    return ATTN_ERR_ALIGN;
  const Range ins[] = {range(dout, qe * es), range(q, qe * es), range(k, ke * es),
                       range(v, ke * es), range(out, qe * es), range(lse, lb)};
  // the static scratch is the library's own memory: no caller buffer meets it
  const Range outs[] = {range(dq, qe * gb), range(dk, ke * gb), range(dv, ke * gb),
                        range(workspace, use_scratch ? 0LL : (long long)need)};
  for (int a = 0; a < 4; ++a) {
    for (const Range& r : ins)
      if (overlap(outs[a], r)) return ATTN_ERR_ALIAS;
    for (int c = a + 1; c < 4; ++c)
      if (overlap(outs[a], outs[c])) return ATTN_ERR_ALIAS;
  }
  (void)hipGetLastError();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (use_scratch && need > 0) {
    st = scratch_for_stream(hs, &workspace);
    if (st != ATTN_OK) return st;
  }
  if (empty) {
    // No queries or no keys: every gradient is zero.  The accumulating form
    // adds nothing; the plain form clears the non-empty gradients (as 32-bit
    // words: d * gb is a multiple of 4).
    if (acc || (qe == 0 && ke == 0)) return ATTN_OK;
    if (qe == 0) {
      hipError_t e = bea::launch_acc_init(static_cast<float*>(dk), nullptr, n, l_k,
                                          h_kv, (int)(d * gb / 4), hs);
      if (e != hipSuccess) return ATTN_ERR_HIP;
      return finish(bea::launch_acc_init(static_cast<float*>(dv), nullptr, n, l_k,
                                         h_kv, (int)(d * gb / 4), hs));
    }
    return finish(bea::launch_acc_init(static_cast<float*>(dq), nullptr, n, l_q, h,
                                       (int)(d * gb / 4), hs));
  }
  AttnShape s{n, l_q, l_k, h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
  mask_bounds(causal, win_l, win_r, q_offset, k_offset, &s.dlo, &s.dhi);
  if (f32)
    return finish(bea::launch_bwd_f32(dout, q, k, v, out, lse, static_cast<float*>(dq),
                                      static_cast<float*>(dk), static_cast<float*>(dv), s,
                                      workspace, acc, prepared, hs));
  if (acc)
    return finish(bea::launch_bwd(dout, q, k, v, out, lse, nullptr, nullptr, nullptr,
                                  s, workspace, true, hs, static_cast<float*>(dq),
                                  static_cast<float*>(dk), static_cast<float*>(dv), prepared));
  return finish(bea::launch_bwd(dout, q, k, v, out, lse, dq, dk, dv, s, workspace,
                                true, hs));
}

}  // namespace

extern "C" {

int attn_bwd(const void* dout, const void* q, const void* k, const void* v,
             const void* out, const float* lse, void* dq, void* dk, void* dv,
             int n, int l_q, int l_k, int h, int h_kv, int d, float scale,
             int causal, int win_l, int win_r, long long q_offset,
             long long k_offset, void* workspace, size_t workspace_bytes,
             void* stream, int dtype) {
  return bwd_entry(dout, q, k, v, out, lse, dq, dk, dv, n, l_q, l_k, h, h_kv, d,
                   scale, causal, win_l, win_r, q_offset, k_offset, workspace,
                   workspace_bytes, stream, dtype, false);
}

int attn_bwd_acc(const void* dout, const void* q, const void* k, const void* v,
                 const void* out, const float* lse, float* dq_acc, float* dk_acc,
                 float* dv_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                 float scale, int causal, int win_l, int win_r, long long q_offset,
                 long long k_offset, void* workspace, size_t workspace_bytes,
                 void* stream, int dtype) {
  return bwd_entry(dout, q, k, v, out, lse, dq_acc, dk_acc, dv_acc, n, l_q, l_k, h,
                   h_kv, d, scale, causal, win_l, win_r, q_offset, k_offset,
                   workspace, workspace_bytes, stream, dtype, true);
}

size_t attn_bwd_prepare_bytes(int n, int l_q, int h) {
  if (!sizes_ok(n, l_q, h, 64)) return 0;
  if ((long long)n * l_q == 0) return 0;
  return bea::bwd_prepared_bytes(n, l_q, h);
}

int attn_bwd_prepare(const void* dout, const void* out, const float* lse, int n, int l_q,
                     int h, int d, void* workspace, size_t workspace_bytes, void* stream,
                     int dtype) {
  // the query-side checks of the backward, with one key/value head
  int st = check_attn_args(n, l_q, 0, h, 1, d, 0.f, dtype);
  if (st != ATTN_OK) return st;
  const long long es = dtype == ATTN_F32 ? 4 : 2;
  const long long qe = (long long)n * l_q * h * d;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(dout, qe) || missing(out, qe) || missing(lse, lb)) return ATTN_ERR_NULL;
  if (qe == 0) return ATTN_OK;
  const size_t need = bea::bwd_prepared_bytes(n, l_q, h);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(dout, 16) || !aligned(out, 16) || !aligned(lse, 4) || !aligned(workspace, 16))
    return ATTN_ERR_ALIGN;
  const Range rw = range(workspace, (long long)need);
  if (overlap(rw, range(dout, qe * es)) || overlap(rw, range(out, qe * es)) ||
      overlap(rw, range(lse, lb)))
    return ATTN_ERR_ALIAS;
  (void)hipGetLastError();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_F32)
    return finish(bea::launch_bwd_f32_prepare(dout, out, lse, n, l_q, h, d, workspace, hs));
  return finish(bea::launch_bwd_prepare(dout, out, lse, n, l_q, h, d, workspace, hs));
}

int attn_bwd_acc_prepared(const void* dout, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, float* dq_acc, float* dk_acc,
                          float* dv_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                          float scale, int causal, int win_l, int win_r, long long q_offset,
                          long long k_offset, void* workspace, size_t workspace_bytes,
                          void* stream, int dtype) {
  return bwd_entry(dout, q, k, v, out, lse, dq_acc, dk_acc, dv_acc, n, l_q, l_k, h, h_kv, d,
                   scale, causal, win_l, win_r, q_offset, k_offset, workspace,
                   workspace_bytes, stream, dtype, true, false, true);
}

int attn_bwd_ring(const void* dout, const void* q, const void* out, const float* lse,
                  const void* const* k_chunks, const void* const* v_chunks,
                  const int* l_k_chunks, const long long* k_offsets,
                  float* const* dk_acc_chunks, float* const* dv_acc_chunks, int n_chunks,
                  void* dq, int n, int l_q, int h, int h_kv, int d, float scale, int causal,
                  int win_l, int win_r, long long q_offset, void* workspace,
                  size_t workspace_bytes, void* stream, int dtype) {
  if (n_chunks < 1 || n_chunks > ATTN_RING_MAX_CHUNKS) return ATTN_ERR_SHAPE;
  if (k_chunks == nullptr || v_chunks == nullptr || l_k_chunks == nullptr ||
      k_offsets == nullptr || dk_acc_chunks == nullptr || dv_acc_chunks == nullptr)
    return ATTN_ERR_NULL;
  for (int c = 0; c < n_chunks; ++c) {
    const int st = check_attn_args(n, l_q, l_k_chunks[c], h, h_kv, d, scale, dtype);
    if (st != ATTN_OK) return st;
  }
  const long long es = dtype == ATTN_F32 ? 4 : 2;
  const long long qe = (long long)n * l_q * h * d;
  const long long lb = (long long)n * h * l_q * 4;
  if (missing(dout, qe) || missing(q, qe) || missing(out, qe) || missing(lse, lb) ||
      missing(dq, qe))
    return ATTN_ERR_NULL;
  bool any_keys = false;
  for (int c = 0; c < n_chunks; ++c) {
    const long long ke = (long long)n * l_k_chunks[c] * h_kv * d;
    if (missing(k_chunks[c], ke) || missing(v_chunks[c], ke) || missing(dk_acc_chunks[c], ke) ||
        missing(dv_acc_chunks[c], ke))
      return ATTN_ERR_NULL;
    any_keys = any_keys || ke > 0;
  }
  const bool work = qe > 0 && any_keys;
  const size_t need = work ? bea::bwd_prepared_bytes(n, l_q, h) : 0;
  if (missing(workspace, (long long)need) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(dout, 16) || !aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(dq, 16) || !aligned(workspace, 16))
    return ATTN_ERR_ALIGN;
  for (int c = 0; c < n_chunks; ++c)
    if (!aligned(k_chunks[c], 16) || !aligned(v_chunks[c], 16) ||
        !aligned(dk_acc_chunks[c], 16) || !aligned(dv_acc_chunks[c], 16))
      return ATTN_ERR_ALIGN;
  // outputs (dq, the workspace, every accumulator) against the inputs and
  // each other
  Range ins[4 + 2 * ATTN_RING_MAX_CHUNKS], outs[2 + 2 * ATTN_RING_MAX_CHUNKS];
  int ni = 0, no = 0;
  ins[ni++] = range(dout, qe * es);
  ins[ni++] = range(q, qe * es);
  ins[ni++] = range(out, qe * es);
  ins[ni++] = range(lse, lb);
  outs[no++] = range(dq, qe * es);
  outs[no++] = range(workspace, (long long)need);
  for (int c = 0; c < n_chunks; ++c) {
    const long long ke = (long long)n * l_k_chunks[c] * h_kv * d;
    ins[ni++] = range(k_chunks[c], ke * es);
    ins[ni++] = range(v_chunks[c], ke * es);
    outs[no++] = range(dk_acc_chunks[c], ke * 4);
    outs[no++] = range(dv_acc_chunks[c], ke * 4);
  }
  for (int a = 0; a < no; ++a) {
    for (int i = 0; i < ni; ++i)
      if (overlap(outs[a], ins[i])) return ATTN_ERR_ALIAS;
    for (int b2 = a + 1; b2 < no; ++b2)
      if (overlap(outs[a], outs[b2])) return ATTN_ERR_ALIAS;
  }
  if (qe == 0) return ATTN_OK;  // no query rows: nothing to write or add
  (void)hipGetLastError();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // no keys in any chunk: dQ = 0 (as 32-bit words), nothing added
  if (!any_keys)
    return finish(bea::launch_acc_init(static_cast<float*>(dq), nullptr, n, l_q, h,
                                       dtype == ATTN_F32 ? d : d / 2, hs));
  if (dtype == ATTN_F32) {
    // float32: dq is its own accumulator (cleared first); D and the base-2
    // LSE prepared once, then one accumulating backward per chunk with keys
    float* dqf = static_cast<float*>(dq);
    hipError_t e = bea::launch_acc_init(dqf, nullptr, n, l_q, h, d, hs);
    if (e == hipSuccess)
      e = bea::launch_bwd_f32_prepare(dout, out, lse, n, l_q, h, d, workspace, hs);
    for (int c = 0; c < n_chunks && e == hipSuccess; ++c) {
      if ((long long)n * l_k_chunks[c] == 0) continue;
      AttnShape sc{n, l_q, l_k_chunks[c], h, h_kv, d, scale, 0, 0, causal ? 1 : 0};
      mask_bounds(causal, win_l, win_r, q_offset, k_offsets[c], &sc.dlo, &sc.dhi);
      e = bea::launch_bwd_f32(dout, q, k_chunks[c], v_chunks[c], out, lse, dqf,
                              dk_acc_chunks[c], dv_acc_chunks[c], sc, workspace, true, true, hs);
    }
    return finish(e);
  }
  bea::BwdChunkArgs ch[bea::kMaxChunks];
  int m = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if ((long long)n * l_k_chunks[c] == 0) continue;
    int dlo, dhi;
    mask_bounds(causal, win_l, win_r, q_offset, k_offsets[c], &dlo, &dhi);
    ch[m++] = bea::BwdChunkArgs{k_chunks[c], v_chunks[c], dk_acc_chunks[c], dv_acc_chunks[c],
                                l_k_chunks[c], dlo, dhi};
  }
  AttnShape s{n, l_q, ch[0].l_k, h, h_kv, d, scale, ch[0].dlo, ch[0].dhi, causal ? 1 : 0};
  return finish(bea::launch_bwd_ring(dout, q, out, lse, ch, m, dq, s, workspace, hs));
}

int attn_bwd_static(const void* dout, const void* q, const void* k, const void* v,
                    const void* out, const float* lse, void* dq, void* dk, void* dv, int n,
                    int l_q, int l_k, int h, int h_kv, int d, float scale, int causal,
                    int win_l, int win_r, long long q_offset, long long k_offset,
                    void* stream, int dtype) {
  return bwd_entry(dout, q, k, v, out, lse, dq, dk, dv, n, l_q, l_k, h, h_kv, d, scale,
                   causal, win_l, win_r, q_offset, k_offset, nullptr, 0, stream, dtype,
                   false, true);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a pointer to a non-empty tensor is NULL";
    case ATTN_ERR_SHAPE: return "invalid sizes (negative, h, h_kv or d <= 0, h % h_kv != 0, or too large)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype or scale";
    case ATTN_ERR_HIP: return "HIP launch failure";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_ALIAS: return "an output overlaps another buffer";
    case ATTN_ERR_ALIGN: return "misaligned tensor pointer";
    default: return "unknown status";
  }
}

}  // extern "C"
