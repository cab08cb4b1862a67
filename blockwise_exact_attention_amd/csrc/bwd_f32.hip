// The float32 backward (dtype ATTN_F32) for gfx950: plain fp32 FMA kernels,
// four lanes per row, for the inputs whose tolerance is 1e-5 (no MFMA form of
// fp32 products is used, so every product and sum is an fp32 FMA).
//
// Sources: "picotron/parallel/context_parallel.py", ring_attention_backward -
// P = exp(S - LSE) from the saved LSE, D = rowsum(dO * O) of the saved output,
// dP = dO V^T, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO; "flash_sharding.py" (flash_attn_jax), ring_bwd - the same
// gradients per key/value chunk, with the global (O, LSE, dO) of the query
// rows, added up over the chunks.
//
//  * bwd_f32_pre: D and LSE * log2(e) per query row (+inf for empty rows),
//    into the same workspace rows the bf16 path uses.
//  * bwd_f32_dkdv: one workgroup per 64 keys of one key/value head, the keys'
//    K and V rows and their dK, dV in registers (four lanes per key, each
//    holding every fourth 16-byte chunk of the row); tiles of 64 query rows
//    of Q and dO stream through LDS for every query head of the group, so the
//    group's sum is formed in the kernel in a fixed order.
//  * bwd_f32_dq: one workgroup per 64 query rows of one head, Q, dO and dQ in
//    registers; tiles of 64 keys of K and V stream through LDS.
// Only the tiles a mask allows are visited.  The ACC instantiations add the
// gradients to the outputs (float32 accumulators) instead of writing them.
#include "common.hpp"
#include "launch.hpp"

namespace bea {
namespace {

constexpr int kF32BwdThreads = 256;
constexpr int kF32BwdRows = kF32BwdThreads / 4;  // rows a workgroup owns
constexpr int kF32BwdTile = 64;                  // rows per streamed tile

struct BwdF32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* lse;
  float* dq;   // written, or (ACC) added to
  float* dk;
  float* dv;
  float* dd;    // D [n, h, l_q]
  float* lse2;  // LSE * log2(e) [n, h, l_q]; +inf for empty rows
  int n, l_q, l_k, h, h_kv, grp;
  float c;      // scale * log2(e) (signed)
  float scale;
  int dlo, dhi;
};

// Dot product of one row pair, each lane holding every fourth 16-byte chunk
// (lane c: chunks c, c + 4, ...), summed over the row's four lanes.
template <int NC>
__device__ __forceinline__ float dot_row(const f32x4_t (&a)[NC], const f32x4_t* b, int c) {
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    const f32x4_t x = b[c + 4 * m];
    s = fmaf(a[m][0], x[0], s);
    s = fmaf(a[m][1], x[1], s);
    s = fmaf(a[m][2], x[2], s);
    s = fmaf(a[m][3], x[3], s);
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  return s;
}

template <int D>
__global__ __launch_bounds__(kF32BwdThreads) void bwd_f32_pre_kernel(BwdF32Params p) {
  constexpr int TPR = D / 4;  // threads per row, one 16-byte chunk each
  const long long rows = (long long)p.n * p.l_q * p.h;
  // a capped grid walks the blocks (one pass on every realistic shape)
  const long long nblocks = (rows * TPR + kF32BwdThreads - 1) / kF32BwdThreads;
  for (long long vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
  const long long row = (vb * kF32BwdThreads + threadIdx.x) / TPR;
  const int part = threadIdx.x % TPR;
  const bool ok = row < rows;
  const long long rr = ok ? row : rows - 1;
  const f32x4_t a = reinterpret_cast<const f32x4_t*>(p.dout + rr * D)[part];
  const f32x4_t b = reinterpret_cast<const f32x4_t*>(p.o + rr * D)[part];
  float acc = a[0] * b[0];
  acc = fmaf(a[1], b[1], acc);
  acc = fmaf(a[2], b[2], acc);
  acc = fmaf(a[3], b[3], acc);
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && part == 0) {
    // rows are ordered (b, i, hq) like O; D and LSE live at [b, hq, i]
    const long long bi = row / p.h;
    const int hq = (int)(row - bi * p.h);
    const long long b = bi / p.l_q;
    const int i = (int)(bi - b * p.l_q);
    const size_t li = ((size_t)b * p.h + hq) * p.l_q + i;
    p.dd[li] = acc;
    const float l = p.lse[li];
    p.lse2[li] = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
  }
  }
}

template <int D, bool ACC>
__global__ __launch_bounds__(kF32BwdThreads) void bwd_f32_dkdv_kernel(BwdF32Params p,
                                                                     int n_ktiles) {
  constexpr int NC = D / 16;  // 16-byte chunks per lane
  constexpr int C4 = D / 4;   // 16-byte chunks per row
  __shared__ f32x4_t qs[kF32BwdTile * C4];
  __shared__ f32x4_t os[kF32BwdTile * C4];
  __shared__ float l2s[kF32BwdTile];
  __shared__ float dds[kF32BwdTile];

  const int tid = threadIdx.x;
  const int c = tid & 3;
  const int kt = blockIdx.x % n_ktiles;
  const int bg = blockIdx.x / n_ktiles;  // b * h_kv + g
  const int b = bg / p.h_kv;
  const int g = bg - b * p.h_kv;
  const int last_key = p.l_k - 1;
  const int j0 = kt * kF32BwdRows;
  const int j = j0 + (tid >> 2);

  const size_t kv_row = (size_t)p.h_kv * D;
  const size_t q_row = (size_t)p.h * D;
  const size_t kv_off = ((size_t)b * p.l_k + min(j, last_key)) * kv_row + (size_t)g * D;
  const f32x4_t* kp = reinterpret_cast<const f32x4_t*>(p.k + kv_off);
  const f32x4_t* vp = reinterpret_cast<const f32x4_t*>(p.v + kv_off);
  f32x4_t kr[NC], vr[NC], dk[NC], dv[NC];
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    kr[m] = kp[c + 4 * m];
    vr[m] = vp[c + 4 * m];
    dk[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // query rows that may see a key of this tile: j - dhi <= i <= j - dlo
  const long long j1 = min(j0 + kF32BwdRows - 1, last_key);
  const long long ilo = max(0LL, (long long)j0 - p.dhi);
  const long long ihi = min((long long)p.l_q - 1, j1 - p.dlo);
  if (ilo <= ihi) {
    for (int hi = 0; hi < p.grp; ++hi) {
      const int hq = g * p.grp + hi;
      const float* qbase = p.q + (size_t)b * p.l_q * q_row + (size_t)hq * D;
      const float* obase = p.dout + (size_t)b * p.l_q * q_row + (size_t)hq * D;
      const size_t lrow = ((size_t)b * p.h + hq) * p.l_q;
      for (long long i0 = (ilo / kF32BwdTile) * kF32BwdTile; i0 <= ihi; i0 += kF32BwdTile) {
        __syncthreads();
        for (int e = tid; e < kF32BwdTile * C4; e += kF32BwdThreads) {
          const int r = e / C4;
          const int c4 = e - r * C4;
          const size_t i = (size_t)min(i0 + r, (long long)p.l_q - 1);
          qs[e] = reinterpret_cast<const f32x4_t*>(qbase + i * q_row)[c4];
          os[e] = reinterpret_cast<const f32x4_t*>(obase + i * q_row)[c4];
        }
        if (tid < kF32BwdTile) {
          const size_t i = (size_t)min(i0 + tid, (long long)p.l_q - 1);
          l2s[tid] = p.lse2[lrow + i];
          dds[tid] = p.dd[lrow + i];
        }
        __syncthreads();
        for (int r = 0; r < kF32BwdTile; ++r) {
          const f32x4_t* qrow = qs + r * C4;
          const f32x4_t* orow = os + r * C4;
          const float s = dot_row<NC>(kr, qrow, c);
          const float dp = dot_row<NC>(vr, orow, c);
          const long long i = i0 + r;
          const long long rel = (long long)j - i;
          const bool ok = i < p.l_q && j <= last_key && rel >= p.dlo && rel <= p.dhi;
          const float pr = ok ? exp2f(fmaf(s, p.c, -l2s[r])) : 0.f;
          const float dsv = pr * (dp - dds[r]);
#pragma unroll
          for (int m = 0; m < NC; ++m) {
            const f32x4_t x = qrow[c + 4 * m];
            const f32x4_t y = orow[c + 4 * m];
            dk[m][0] = fmaf(dsv, x[0], dk[m][0]);
            dk[m][1] = fmaf(dsv, x[1], dk[m][1]);
            dk[m][2] = fmaf(dsv, x[2], dk[m][2]);
            dk[m][3] = fmaf(dsv, x[3], dk[m][3]);
            dv[m][0] = fmaf(pr, y[0], dv[m][0]);
            dv[m][1] = fmaf(pr, y[1], dv[m][1]);
            dv[m][2] = fmaf(pr, y[2], dv[m][2]);
            dv[m][3] = fmaf(pr, y[3], dv[m][3]);
          }
        }
      }
    }
  }
  if (j <= last_key) {
    const size_t off = ((size_t)b * p.l_k + j) * kv_row + (size_t)g * D;
    f32x4_t* dkp = reinterpret_cast<f32x4_t*>(p.dk + off);
    f32x4_t* dvp = reinterpret_cast<f32x4_t*>(p.dv + off);
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const f32x4_t x = dk[m] * p.scale;
      if (ACC) {
        dkp[c + 4 * m] += x;
        dvp[c + 4 * m] += dv[m];
      } else {
        dkp[c + 4 * m] = x;
        dvp[c + 4 * m] = dv[m];
      }
    }
  }
}

template <int D, bool ACC>
__global__ __launch_bounds__(kF32BwdThreads) void bwd_f32_dq_kernel(BwdF32Params p,
                                                                   int n_qtiles) {
  constexpr int NC = D / 16;
  constexpr int C4 = D / 4;
  __shared__ f32x4_t ks[kF32BwdTile * C4];
  __shared__ f32x4_t vs[kF32BwdTile * C4];

  const int tid = threadIdx.x;
  const int c = tid & 3;
  const int qt = blockIdx.x % n_qtiles;
  const int bh = blockIdx.x / n_qtiles;  // b * h + hq
  const int b = bh / p.h;
  const int hq = bh - b * p.h;
  const int g = hq / p.grp;
  const int last_row = p.l_q - 1;
  const int i0 = qt * kF32BwdRows;
  const int i = i0 + (tid >> 2);

  const size_t q_row = (size_t)p.h * D;
  const size_t kv_row = (size_t)p.h_kv * D;
  const size_t q_off = ((size_t)b * p.l_q + min(i, last_row)) * q_row + (size_t)hq * D;
  const f32x4_t* qp = reinterpret_cast<const f32x4_t*>(p.q + q_off);
  const f32x4_t* op = reinterpret_cast<const f32x4_t*>(p.dout + q_off);
  f32x4_t qr[NC], orr[NC], dq[NC];
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    qr[m] = qp[c + 4 * m];
    orr[m] = op[c + 4 * m];
    dq[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const size_t li = ((size_t)b * p.h + hq) * p.l_q + min(i, last_row);
  const float l2 = p.lse2[li];
  const float dd = p.dd[li];

  const float* kbase = p.k + (size_t)b * p.l_k * kv_row + (size_t)g * D;
  const float* vbase = p.v + (size_t)b * p.l_k * kv_row + (size_t)g * D;
  // keys that a row of this tile may see: i + dlo <= j <= i + dhi
  const long long jlo = max(0LL, (long long)i0 + p.dlo);
  const long long jhi = min((long long)p.l_k - 1,
                            (long long)min(i0 + kF32BwdRows - 1, last_row) + p.dhi);
  if (jlo <= jhi) {
    for (long long j0 = (jlo / kF32BwdTile) * kF32BwdTile; j0 <= jhi; j0 += kF32BwdTile) {
      __syncthreads();
      for (int e = tid; e < kF32BwdTile * C4; e += kF32BwdThreads) {
        const int r = e / C4;
        const int c4 = e - r * C4;
        const size_t j = (size_t)min(j0 + r, (long long)p.l_k - 1);
        ks[e] = reinterpret_cast<const f32x4_t*>(kbase + j * kv_row)[c4];
        vs[e] = reinterpret_cast<const f32x4_t*>(vbase + j * kv_row)[c4];
      }
      __syncthreads();
      for (int r = 0; r < kF32BwdTile; ++r) {
        const f32x4_t* krow = ks + r * C4;
        const float s = dot_row<NC>(qr, krow, c);
        const float dp = dot_row<NC>(orr, vs + r * C4, c);
        const long long j = j0 + r;
        const long long rel = j - i;
        const bool ok = j < p.l_k && i <= last_row && rel >= p.dlo && rel <= p.dhi;
        const float pr = ok ? exp2f(fmaf(s, p.c, -l2)) : 0.f;
        const float dsv = pr * (dp - dd);
#pragma unroll
        for (int m = 0; m < NC; ++m) {
          const f32x4_t x = krow[c + 4 * m];
          dq[m][0] = fmaf(dsv, x[0], dq[m][0]);
          dq[m][1] = fmaf(dsv, x[1], dq[m][1]);
          dq[m][2] = fmaf(dsv, x[2], dq[m][2]);
          dq[m][3] = fmaf(dsv, x[3], dq[m][3]);
        }
      }
    }
  }
  if (i <= last_row) {
    f32x4_t* dqp = reinterpret_cast<f32x4_t*>(p.dq + ((size_t)b * p.l_q + i) * q_row +
                                              (size_t)hq * D);
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const f32x4_t x = dq[m] * p.scale;
      if (ACC) dqp[c + 4 * m] += x;
      else dqp[c + 4 * m] = x;
    }
  }
}

template <int D>
void launch_f32_pre_d(const BwdF32Params& p, hipStream_t stream) {
  const long long rows = (long long)p.n * p.l_q * p.h;
  const long long blocks = (rows * (D / 4) + kF32BwdThreads - 1) / kF32BwdThreads;
  hipLaunchKernelGGL((bwd_f32_pre_kernel<D>), dim3(capped_grid(blocks)), dim3(kF32BwdThreads), 0,
                     stream, p);
}

template <int D, bool ACC>
void launch_f32_grads_d(const BwdF32Params& p, hipStream_t stream) {
  const int n_ktiles = (p.l_k + kF32BwdRows - 1) / kF32BwdRows;
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, ACC>),
                     dim3((unsigned)((long long)n_ktiles * p.n * p.h_kv)),
                     dim3(kF32BwdThreads), 0, stream, p, n_ktiles);
  const int n_qtiles = (p.l_q + kF32BwdRows - 1) / kF32BwdRows;
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D, ACC>),
                     dim3((unsigned)((long long)n_qtiles * p.n * p.h)),
                     dim3(kF32BwdThreads), 0, stream, p, n_qtiles);
}

}  // namespace

hipError_t launch_bwd_f32_prepare(const void* dout, const void* out, const float* lse, int n,
                                  int l_q, int h, int d, void* workspace, hipStream_t stream) {
  BwdF32Params p{};
  p.dout = static_cast<const float*>(dout);
  p.o = static_cast<const float*>(out);
  p.lse = lse;
  bwd_prepared_rows(workspace, n, l_q, h, &p.dd, &p.lse2);
  p.n = n;
  p.l_q = l_q;
  p.h = h;
  if (d == 128) launch_f32_pre_d<128>(p, stream);
  else launch_f32_pre_d<64>(p, stream);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const void* dout, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, float* dq, float* dk, float* dv,
                          const AttnShape& s, void* workspace, bool acc, bool prepared,
                          hipStream_t stream) {
  BwdF32Params p{};
  p.q = static_cast<const float*>(q);
  p.k = static_cast<const float*>(k);
  p.v = static_cast<const float*>(v);
  p.o = static_cast<const float*>(out);
  p.dout = static_cast<const float*>(dout);
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  bwd_prepared_rows(workspace, s.n, s.l_q, s.h, &p.dd, &p.lse2);
  p.n = s.n;
  p.l_q = s.l_q;
  p.l_k = s.l_k;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  p.c = s.scale * kLog2e;
  p.scale = s.scale;
  p.dlo = s.dlo;
  p.dhi = s.dhi;
  if (s.d == 128) {
    if (!prepared) launch_f32_pre_d<128>(p, stream);
    if (acc) launch_f32_grads_d<128, true>(p, stream);
    else launch_f32_grads_d<128, false>(p, stream);
  } else {
    if (!prepared) launch_f32_pre_d<64>(p, stream);
    if (acc) launch_f32_grads_d<64, true>(p, stream);
    else launch_f32_grads_d<64, false>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace bea
