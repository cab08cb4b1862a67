// Exact attention backward for gfx950 (bf16 MFMA, fp32 accumulation), by
// recomputation from the saved LSE.
//
// What is computed follows "picotron/parallel/context_parallel.py",
// ring_attention_backward: P = exp(S - LSE); dV = P^T dO; dP = dO V^T;
// D = rowsum(dO * O); dS = P * (dP - D), zero where masked;
// dQ = scale dS K; dK = scale dS^T Q.  Grouped heads (RingAttention._repeat_kv)
// make dK and dV of a key/value head the sum over the query heads that read
// it.  Gradients are written in the input dtype ("flash_sharding.py",
// ring_bwd casts them to q's dtype).
//
// Three kernels, no atomics (results are bitwise repeatable):
//  * bwd_pre: D_i and LSE_i * log2(e) per query row (+inf for a row with no
//    allowed key, so its P is exactly 0), into the workspace.
//  * bwd_dkdv: one workgroup per 128 keys of one key/value head, 32 keys per
//    wave held in VGPRs (B operand); query tiles of the whole group stream
//    through LDS.  S = Q K^T and dP = dO V^T come out with one key per lane,
//    which is exactly the B-operand layout dV^T += dO^T P and
//    dK^T += Q^T dS need, so P and dS never leave registers; dO^T and Q^T are
//    staged transposed in LDS.
//  * bwd_dq: one workgroup per 128 query rows of one head, Q and dO resident
//    (B operands); key tiles stream through LDS.  S^T = K Q^T and
//    dP^T = V dO^T put one query per lane, so dQ^T += K^T dS^T reads dS^T
//    straight from registers; K^T is staged transposed in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace bea {
namespace {

constexpr int kThreads = 256;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dd;    // D [n, h, l_q]
  float* lse2;  // LSE * log2(e) [n, h, l_q]; +inf for empty rows
  int n, l_q, l_k, h, h_kv, grp;
  float c;      // scale * log2(e) (signed)
  float scale;
  int dlo, dhi;
};

// Position of row rr inside a transposed LDS row: the same in-16 permutation
// as the forward's V^T (bits 2 and 3 swap), so a lane of half h reads its 8
// k-slots {4h+0..3, 8+4h+0..3} as one 16-byte access.
__device__ __forceinline__ int tr_pos(int rr) {
  return (rr & ~12) | ((rr & 4) << 1) | ((rr & 8) >> 1);
}

// Copy a [ROWS x D] bf16 tile (row r at base + (r0 + r) * stride, rows
// clamped to limit - 1) into LDS: row-major with row stride D + 8 when RM,
// and transposed (dim-major, rows permuted by tr_pos, row stride ROWS + 8)
// when TR.  Each thread moves groups of 4 rows x 8 dims.
template <int ROWS, int D, bool RM, bool TR>
__device__ __forceinline__ void tile_to_lds(const uint16_t* base, size_t stride,
                                            int r0, int limit, uint16_t* rm,
                                            uint16_t* tr) {
  constexpr int GROUPS = (ROWS / 4) * (D / 8);
  for (int gi = threadIdx.x; gi < GROUPS; gi += kThreads) {
    const int rg = gi / (D / 8);
    const int c8 = gi - rg * (D / 8);
    u32x4_t x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(r0 + 4 * rg + r, limit - 1);
      x[r] = *reinterpret_cast<const u32x4_t*>(base + (size_t)row * stride + c8 * 8);
    }
    if (RM) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4_t*>(&rm[(4 * rg + r) * (D + 8) + c8 * 8]) = x[r];
    }
    if (TR) {
      const int pos = tr_pos(4 * rg);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        const int sh = (dd & 1) * 16;
        u32x2_t pk;
        pk[0] = ((x[0][w] >> sh) & 0xffffu) | (((x[1][w] >> sh) & 0xffffu) << 16);
        pk[1] = ((x[2][w] >> sh) & 0xffffu) | (((x[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2_t*>(&tr[(c8 * 8 + dd) * (ROWS + 8) + pos]) = pk;
      }
    }
  }
}

// ------------------------------------------------------------ preprocess

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;  // threads per row
  const long long rows = (long long)p.n * p.l_q * p.h;
  const long long row = ((long long)blockIdx.x * kThreads + threadIdx.x) / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  const bool ok = row < rows;
  const long long rr = ok ? row : rows - 1;
  {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p.dout + rr * D + part * 8);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p.o + rr * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_lo(a[w]), bf16_lo(b[w]), acc);
      acc = fmaf(bf16_hi(a[w]), bf16_hi(b[w]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && part == 0) {
    // row order (b, i, hq); D and LSE live at [b, hq, i]
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

// ------------------------------------------------------------ dK, dV

constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWG = 4 * kKeysPerWave;

template <int D>
struct __attribute__((aligned(16))) DkdvSmem {
  static constexpr int BQ = 8192 / D;  // query rows per step (64 or 128)
  uint16_t q[BQ * (D + 8)];
  uint16_t qt[D * (BQ + 8)];
  uint16_t dout[BQ * (D + 8)];
  uint16_t doutt[D * (BQ + 8)];
  float lse2[BQ];
  float dd[BQ];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p, int n_ktiles,
                                                               int reverse) {
  constexpr int BQ = DkdvSmem<D>::BQ;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = BQ / 32;
  constexpr int NPS = BQ / 16;
  constexpr int RS = D + 8;
  constexpr int TS = BQ + 8;
  __shared__ DkdvSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // blockIdx.x -> (key tile, b * h_kv + g); under causal masking the first
  // key tiles are read by the most query rows: they go first
  const int heads = p.n * p.h_kv;
  const int rank = blockIdx.x / heads;
  const int kvh = blockIdx.x - rank * heads;
  const int kt = reverse ? rank : n_ktiles - 1 - rank;
  const int b = kvh / p.h_kv;
  const int g = kvh - b * p.h_kv;
  const int k0 = kt * kKeysPerWG;
  const int kw = k0 + wave * kKeysPerWave;
  const int last_key = p.l_k - 1;
  const int kj = kw + col;  // this lane's key (as B-operand column)

  const size_t kv_row = (size_t)p.h_kv * D;
  const size_t q_row = (size_t)p.h * D;
  // resident K and V rows of the wave's 32 keys
  u32x4_t kf[NDS], vf[NDS];
  {
    const size_t off = ((size_t)b * p.l_k + min(kj, last_key)) * kv_row +
                       (size_t)g * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      kf[s] = *reinterpret_cast<const u32x4_t*>(p.k + off + 16 * s);
      vf[s] = *reinterpret_cast<const u32x4_t*>(p.v + off + 16 * s);
    }
  }
  f32x16_t dkt[NDB], dvt[NDB];  // dK^T, dV^T: lane = key, regs = dims
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkt[db][r] = 0.f;
      dvt[db][r] = 0.f;
    }

  // query rows that may see any key of this workgroup / wave
  const int kb_last = min(k0 + kKeysPerWG - 1, last_key);
  const long long qlo = max(0LL, (long long)k0 - p.dhi);
  const long long qhi = min((long long)p.l_q - 1, (long long)kb_last - p.dlo);
  const bool wave_live = kw <= last_key;
  const int kw_last = min(kw + kKeysPerWave - 1, last_key);

  if (qlo <= qhi) {
    const int t_begin = (int)(qlo / BQ);
    const int t_end = (int)(qhi / BQ) + 1;
    for (int hq = g * p.grp; hq < (g + 1) * p.grp; ++hq) {
      const size_t rowbase = (size_t)b * p.l_q * q_row + (size_t)hq * D;
      const size_t lbase = ((size_t)b * p.h + hq) * p.l_q;
      for (int t = t_begin; t < t_end; ++t) {
        const int i0 = t * BQ;
        __syncthreads();
        tile_to_lds<BQ, D, true, true>(p.q + rowbase, q_row, i0, p.l_q, sm.q, sm.qt);
        tile_to_lds<BQ, D, true, true>(p.dout + rowbase, q_row, i0, p.l_q, sm.dout,
                                       sm.doutt);
        if (tid < BQ) {
          const int i = min(i0 + tid, p.l_q - 1);
          sm.lse2[tid] = p.lse2[lbase + i];
          sm.dd[tid] = p.dd[lbase + i];
        }
        __syncthreads();
        const int i_last = min(i0 + BQ - 1, p.l_q - 1);
        const bool live = wave_live && (long long)kw_last - i0 >= p.dlo &&
                          (long long)kw - i_last <= p.dhi;
        if (!live) continue;
        const bool full = (i0 + BQ <= p.l_q) && (kw + kKeysPerWave <= p.l_k) &&
                          ((long long)kw - (i0 + BQ - 1) >= p.dlo) &&
                          ((long long)(kw + kKeysPerWave - 1) - i0 <= p.dhi);
        // S = Q K^T and dP = dO V^T: [32 queries x 32 keys] blocks, lane = key
        f32x16_t sa[NQB], dpa[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sa[qb][r] = 0.f;
            dpa[qb][r] = 0.f;
          }
#pragma unroll
          for (int s = 0; s < NDS; ++s) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                &sm.q[(32 * qb + col) * RS + 16 * s + 8 * half]);
            sa[qb] = mfma32x32x16(a, kf[s], sa[qb]);
            const u32x4_t a2 = *reinterpret_cast<const u32x4_t*>(
                &sm.dout[(32 * qb + col) * RS + 16 * s + 8 * half]);
            dpa[qb] = mfma32x32x16(a2, vf[s], dpa[qb]);
          }
        }
        // P = exp2(c s - lse2), dS = P (dP - D); both packed to bf16
        u32x4_t pp[NPS], dsp[NPS];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int qi_loc = 32 * qb + 8 * r4 + 4 * half;
            const f32x4_t l2 = *reinterpret_cast<const f32x4_t*>(&sm.lse2[qi_loc]);
            const f32x4_t dv = *reinterpret_cast<const f32x4_t*>(&sm.dd[qi_loc]);
            float pv[4], dsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * r4 + e;
              float pe = __builtin_amdgcn_exp2f(fmaf(sa[qb][r], p.c, -l2[e]));
              if (!full) {
                const int i = i0 + qi_loc + e;
                const int rel = kj - i;
                const bool ok = rel >= p.dlo && rel <= p.dhi && i < p.l_q &&
                                kj < p.l_k;
                pe = ok ? pe : 0.f;
              }
              pv[e] = pe;
              dsv[e] = pe * (dpa[qb][r] - dv[e]);
            }
            const int t16 = 2 * qb + (r4 >> 1);
            const int w0 = (r4 & 1) * 2;
            pp[t16][w0] = pack_bf16x2(pv[0], pv[1]);
            pp[t16][w0 + 1] = pack_bf16x2(pv[2], pv[3]);
            dsp[t16][w0] = pack_bf16x2(dsv[0], dsv[1]);
            dsp[t16][w0 + 1] = pack_bf16x2(dsv[2], dsv[3]);
          }
        // dV^T += dO^T P ; dK^T += Q^T dS   (k-slots = query rows)
#pragma unroll
        for (int t16 = 0; t16 < NPS; ++t16)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4_t ad = *reinterpret_cast<const u32x4_t*>(
                &sm.doutt[(32 * db + col) * TS + 16 * t16 + 8 * half]);
            dvt[db] = mfma32x32x16(ad, pp[t16], dvt[db]);
            const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(
                &sm.qt[(32 * db + col) * TS + 16 * t16 + 8 * half]);
            dkt[db] = mfma32x32x16(aq, dsp[t16], dkt[db]);
          }
      }
    }
  }

  if (kj <= last_key) {
    const size_t off = ((size_t)b * p.l_k + kj) * kv_row + (size_t)g * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * half;
        u32x2_t wk, wv;
        wk[0] = pack_bf16x2(dkt[db][4 * r4] * p.scale, dkt[db][4 * r4 + 1] * p.scale);
        wk[1] = pack_bf16x2(dkt[db][4 * r4 + 2] * p.scale, dkt[db][4 * r4 + 3] * p.scale);
        wv[0] = pack_bf16x2(dvt[db][4 * r4], dvt[db][4 * r4 + 1]);
        wv[1] = pack_bf16x2(dvt[db][4 * r4 + 2], dvt[db][4 * r4 + 3]);
        *reinterpret_cast<u32x2_t*>(p.dk + off + dim) = wk;
        *reinterpret_cast<u32x2_t*>(p.dv + off + dim) = wv;
      }
  }
}

// ------------------------------------------------------------ dQ

template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int BN = 8192 / D;  // keys per step (64 or 128)
  uint16_t k[BN * (D + 8)];
  uint16_t kt[D * (BN + 8)];
  uint16_t v[BN * (D + 8)];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p, int n_qtiles,
                                                             int reverse) {
  constexpr int BN = DqSmem<D>::BN;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  constexpr int NPS = BN / 16;
  constexpr int RS = D + 8;
  constexpr int TS = BN + 8;
  constexpr int BM = 128;
  __shared__ DqSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int heads = p.n * p.h;
  const int rank = blockIdx.x / heads;
  const int head = blockIdx.x - rank * heads;
  const int tile = reverse ? n_qtiles - 1 - rank : rank;
  const int b = head / p.h;
  const int hq = head - b * p.h;
  const int g = hq / p.grp;
  const int last_row = p.l_q - 1;
  const int i0 = tile * BM;
  const int iw = i0 + 32 * wave;
  const int qi = iw + col;

  const size_t q_row = (size_t)p.h * D;
  const size_t kv_row = (size_t)p.h_kv * D;
  u32x4_t qf[NDS], dof[NDS];
  {
    const size_t off = ((size_t)b * p.l_q + min(qi, last_row)) * q_row +
                       (size_t)hq * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      qf[s] = *reinterpret_cast<const u32x4_t*>(p.q + off + 16 * s);
      dof[s] = *reinterpret_cast<const u32x4_t*>(p.dout + off + 16 * s);
    }
  }
  const size_t li = ((size_t)b * p.h + hq) * p.l_q + min(qi, last_row);
  const float l2 = p.lse2[li];
  const float dval = p.dd[li];

  f32x16_t dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;

  const long long jlo = max(0LL, (long long)i0 + p.dlo);
  const long long jhi = min((long long)p.l_k - 1,
                            (long long)min(i0 + BM - 1, last_row) + p.dhi);
  const int wa = iw;
  const int wb = min(iw + 31, last_row);
  const bool wave_live = wa <= last_row;
  const long long wjlo = max(0LL, (long long)wa + p.dlo);
  const long long wjhi = min((long long)p.l_k - 1, (long long)wb + p.dhi);
  const uint16_t* kbase = p.k + (size_t)b * p.l_k * kv_row + (size_t)g * D;
  const uint16_t* vbase = p.v + (size_t)b * p.l_k * kv_row + (size_t)g * D;

  if (jlo <= jhi) {
    const int kt_begin = (int)(jlo / BN);
    const int kt_end = (int)(jhi / BN) + 1;
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int j0 = kt * BN;
      __syncthreads();
      tile_to_lds<BN, D, true, true>(kbase, kv_row, j0, p.l_k, sm.k, sm.kt);
      tile_to_lds<BN, D, true, false>(vbase, kv_row, j0, p.l_k, sm.v, nullptr);
      __syncthreads();
      const bool live = wave_live && (long long)j0 <= wjhi &&
                        (long long)(j0 + BN - 1) >= wjlo;
      if (!live) continue;
      const bool full = (j0 + BN <= p.l_k) && ((long long)j0 - wb >= p.dlo) &&
                        ((long long)(j0 + BN - 1) - wa <= p.dhi);
      f32x16_t sa[NKB], dpa[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sa[kb][r] = 0.f;
          dpa[kb][r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              &sm.k[(32 * kb + col) * RS + 16 * s + 8 * half]);
          sa[kb] = mfma32x32x16(a, qf[s], sa[kb]);
          const u32x4_t a2 = *reinterpret_cast<const u32x4_t*>(
              &sm.v[(32 * kb + col) * RS + 16 * s + 8 * half]);
          dpa[kb] = mfma32x32x16(a2, dof[s], dpa[kb]);
        }
      }
      u32x4_t dsp[NPS];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float ds2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float pe = __builtin_amdgcn_exp2f(fmaf(sa[kb][r + e], p.c, -l2));
            if (!full) {
              const int j = j0 + 32 * kb + 8 * ((r + e) >> 2) + 4 * half + ((r + e) & 3);
              const int rel = j - qi;
              const bool ok = rel >= p.dlo && rel <= p.dhi && j < p.l_k;
              pe = ok ? pe : 0.f;
            }
            ds2[e] = pe * (dpa[kb][r + e] - dval);
          }
          dsp[2 * kb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(ds2[0], ds2[1]);
        }
      // dQ^T += K^T dS^T   (k-slots = keys)
#pragma unroll
      for (int t16 = 0; t16 < NPS; ++t16)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              &sm.kt[(32 * db + col) * TS + 16 * t16 + 8 * half]);
          dqt[db] = mfma32x32x16(a, dsp[t16], dqt[db]);
        }
    }
  }

  if (qi <= last_row) {
    uint16_t* optr = p.dq + ((size_t)b * p.l_q + qi) * q_row + (size_t)hq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * db + 8 * r4 + 4 * half;
        u32x2_t w;
        w[0] = pack_bf16x2(dqt[db][4 * r4] * p.scale, dqt[db][4 * r4 + 1] * p.scale);
        w[1] = pack_bf16x2(dqt[db][4 * r4 + 2] * p.scale, dqt[db][4 * r4 + 3] * p.scale);
        *reinterpret_cast<u32x2_t*>(optr + dim) = w;
      }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, int causal, hipStream_t stream) {
  const long long rows = (long long)p.n * p.l_q * p.h;
  const long long pre_blocks = (rows * (D / 8) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_blocks), dim3(kThreads),
                     0, stream, p);
  const int n_ktiles = (p.l_k + kKeysPerWG - 1) / kKeysPerWG;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>),
                     dim3((unsigned)(n_ktiles * p.n * p.h_kv)), dim3(kThreads), 0,
                     stream, p, n_ktiles, causal ? 1 : 0);
  const int n_qtiles = (p.l_q + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(n_qtiles * p.n * p.h)),
                     dim3(kThreads), 0, stream, p, n_qtiles, causal ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int n, int l_q, int h) {
  // D and LSE*log2(e), one float each per query row
  return (size_t)2 * n * l_q * h * sizeof(float);
}

hipError_t launch_bwd(const void* dout, const void* q, const void* k,
                      const void* v, const void* out, const float* lse,
                      void* dq, void* dk, void* dv, const AttnShape& s,
                      void* workspace, bool bf16, hipStream_t stream) {
  if (!bf16) return hipErrorNotSupported;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  const size_t rows = (size_t)s.n * s.l_q * s.h;
  p.dd = static_cast<float*>(workspace);
  p.lse2 = static_cast<float*>(workspace) + rows;
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
  return s.d == 128 ? launch_bwd_d<128>(p, s.causal, stream)
                    : launch_bwd_d<64>(p, s.causal, stream);
}

}  // namespace bea
