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
// Three kernels (four when the dK/dV grid is split), no atomics, results
// bitwise repeatable:
//  * bwd_pre: D_i and LSE_i * log2(e) per query row (+inf for a row with no
//    allowed key, so its P is exactly 0), into the workspace.
//  * bwd_dkdv: one workgroup per 128 keys of one key/value head, 32 keys per
//    wave held in VGPRs (B operand); query tiles of the whole group stream
//    through LDS.  S = Q K^T and dP = dO V^T come out with one key per lane,
//    which is exactly the B-operand layout dV^T += dO^T P and
//    dK^T += Q^T dS need, so P and dS never leave registers; dO^T and Q^T are
//    read transposed out of the row-major tiles.
//  * bwd_dq: one workgroup per 128 query rows of one head, Q and dO resident
//    (B operands); key tiles stream through LDS.  S^T = K Q^T and
//    dP^T = V dO^T put one query per lane, so dQ^T += K^T dS^T reads dS^T
//    straight from registers; K^T is read transposed out of the K tile.  On
//    a small grid (under two workgroups per CU) a workgroup has two groups
//    of four waves taking alternate key tiles, whose dQ^T partials are added
//    through LDS.
//  * bwd_dkdv_reduce (small dK/dV grids only): the sum of the per-slice dK,
//    dV partials, in slice order.
// The ACC instantiations add the gradients to float32 accumulators instead of
// writing them (one step of the ring backward).  Tiles use the layout of the
// forward kernel (swizzled rows, direct loads one tile ahead).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace bea {
namespace {

constexpr int kThreads = 256;

// One key/value chunk of the multi-chunk (ring share) kernels: its tensors,
// its fp32 dK/dV accumulators, its mask bounds, its 128-key tiles and the
// first dK/dV workgroup id that serves it.
struct BwdChunk {
  const uint16_t* k;
  const uint16_t* v;
  float* dk_acc;
  float* dv_acc;
  int l_k, dlo, dhi;
  int ktiles;
  int wg_begin;
};

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
  float* dq_acc;  // ACC kernels: fp32 accumulators the gradients are added to
  float* dk_acc;
  float* dv_acc;
  float* part;      // split dK/dV: per-slice fp32 partials (dK at part, dV
  size_t part_half; //   part_half floats later), each [n, l_k, h_kv, d]
  int split;        // slices of the query steps per key tile (1: no split)
  float* dd;    // D [n, h, l_q]
  float* lse2;  // LSE * log2(e) [n, h, l_q]; +inf for empty rows
  int n, l_q, l_k, h, h_kv, grp;
  float c;      // scale * log2(e) (signed)
  float scale;
  int dlo, dhi;
  // MULTI kernels: the chunks (the single-chunk fields above are unused)
  BwdChunk ch[kMaxChunks];
  int n_chunks;
};

// ------------------------------------------------------------ preprocess

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;  // threads per row
  const long long rows = (long long)p.n * p.l_q * p.h;
  // a capped grid walks the blocks (one pass on every realistic shape)
  const long long nblocks = (rows * TPR + kThreads - 1) / kThreads;
  for (long long vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
  const long long row = (vb * kThreads + threadIdx.x) / TPR;
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
}

// ------------------------------------------------------------ dK, dV
//
// One workgroup per 128 keys of one key/value head, 4 waves x 32 keys; the
// wave's K and V rows stay in VGPRs as B operands.  For every query head of
// the group, tiles of 64 query rows of Q and dO stream through LDS (swizzled
// rows, three buffer sets, loaded one tile ahead by direct buffer loads) with
// their LSE * log2(e) and D entries.  Per tile: S = Q K^T and dP = dO V^T (Q
// and dO rows as A operands) come out with one key per lane and one query
// per k-slot position, which is the B layout of dV^T += dO^T P and
// dK^T += Q^T dS, so P and dS stay in registers; dO^T and Q^T are read
// transposed out of the row-major tiles.
//
// With one wave per SIMD nothing else hides a wave's own latencies, so the
// step is software-pipelined: the dV/dK products of tile u - 1 (its P and dS
// kept in registers, its Q and dO still in the third buffer set) are issued
// at step u, their transposed operands read three products ahead, with the
// softmax of tile u split into chunks placed between them.  Each chunk is
// pinned there by an empty asm on its results; left alone, the compiler
// sinks all exponentials below the last product and the step runs ~11%
// slower on a 16384-token causal backward.

constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWG = 4 * kKeysPerWave;

template <int D, bool ACC, bool MULTI>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p, int n_ktiles,
                                                               int reverse) {
  static_assert(!MULTI || ACC, "the multi-chunk form accumulates");
  // MULTI: workgroups are numbered chunk by chunk; this one's chunk supplies
  // the key side (tensors, accumulators, length, mask bounds, tiles)
  // (kept in locals: p itself is never written, so that the chunk table is
  // read from the kernel arguments instead of a private copy)
  int wg = blockIdx.x;
  const uint16_t* kp_ = p.k;
  const uint16_t* vp_ = p.v;
  float* dka_ = p.dk_acc;
  float* dva_ = p.dv_acc;
  int lk_ = p.l_k, dlo_ = p.dlo, dhi_ = p.dhi;
  if constexpr (MULTI) {
    int c = 0;
    while (c + 1 < p.n_chunks && wg >= p.ch[c + 1].wg_begin) ++c;
    wg -= p.ch[c].wg_begin;
    n_ktiles = p.ch[c].ktiles;
    kp_ = p.ch[c].k;
    vp_ = p.ch[c].v;
    dka_ = p.ch[c].dk_acc;
    dva_ = p.ch[c].dv_acc;
    lk_ = p.ch[c].l_k;
    dlo_ = p.ch[c].dlo;
    dhi_ = p.ch[c].dhi;
  }
  constexpr int BQ = 64;         // query rows per tile
  constexpr int RB = D * 2;      // bytes per tile row
  constexpr int TB = BQ * RB;    // bytes per tile
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = BQ / 32;
  constexpr int NPS = BQ / 16;
  constexpr uint32_t kVC = D == 128 ? 32u : 16u;
  __shared__ __attribute__((aligned(16))) unsigned char q_lds0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char q_lds1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char o_lds0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char o_lds1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char q_lds2[TB];
  __shared__ __attribute__((aligned(16))) unsigned char o_lds2[TB];
  __shared__ __attribute__((aligned(16))) float l_lds0[2 * BQ];  // LSE2 then D
  __shared__ __attribute__((aligned(16))) float l_lds1[2 * BQ];
  __shared__ __attribute__((aligned(16))) float l_lds2[2 * BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // blockIdx.x -> (slice, key tile, b * h_kv + g); under causal masking the
  // first key tiles are read by the most query rows: they go first
  const int heads = p.n * p.h_kv;
  const int tiles_heads = n_ktiles * heads;
  const int slice = wg / tiles_heads;
  const int wid = wg - slice * tiles_heads;
  const int rank = wid / heads;
  const int kvh = wid - rank * heads;
  const int kt = reverse ? rank : n_ktiles - 1 - rank;
  const int b = kvh / p.h_kv;
  const int g = kvh - b * p.h_kv;
  const int k0 = kt * kKeysPerWG;
  const int kw = k0 + wave * kKeysPerWave;
  const int last_key = lk_ - 1;
  const int kj = kw + col;  // this lane's key (as B-operand column)

  const size_t kv_row = (size_t)p.h_kv * D;
  const size_t q_row = (size_t)p.h * D;
  const uint32_t q_row_b = (uint32_t)q_row * 2u;
  // resident K and V rows of the wave's 32 keys
  u32x4_t kf[NDS], vf[NDS];
  {
    const size_t off = ((size_t)b * lk_ + min(kj, last_key)) * kv_row +
                       (size_t)g * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      kf[s] = *reinterpret_cast<const u32x4_t*>(kp_ + off + 16 * s);
      vf[s] = *reinterpret_cast<const u32x4_t*>(vp_ + off + 16 * s);
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
  const long long qlo = max(0LL, (long long)k0 - dhi_);
  const long long qhi = min((long long)p.l_q - 1, (long long)kb_last - dlo_);
  const bool wave_live = kw <= last_key;
  const int kw_last = min(kw + kKeysPerWave - 1, last_key);

  const uint32_t lane_off = tile_lane_offset<D>(wave, lane, q_row_b);
  uint32_t ka0, va0;
  lds_read_bases<D>(lane, ka0, va0);

  // steps u = (query head of the group, query tile) flattened
  const int t_begin = qlo <= qhi ? (int)(qlo / BQ) : 0;
  const int nt = qlo <= qhi ? (int)(qhi / BQ) + 1 - t_begin : 0;
  const int n_steps = nt * p.grp;
  // this workgroup's slice of the steps
  const int u_lo = (int)((long long)slice * n_steps / p.split);
  const int u_end = (int)((long long)(slice + 1) * n_steps / p.split);
  auto load = [&](int u, unsigned char* qd, unsigned char* od, float* ld) {
    const int hq = g * p.grp + u / nt;
    const int i0 = (t_begin + u % nt) * BQ;
    const size_t rowbase = (size_t)b * p.l_q * q_row + (size_t)hq * D;
    tile_dma<D>(p.q + rowbase, i0, (long long)p.l_q - i0, q_row_b, qd, wave, lane_off);
    tile_dma<D>(p.dout + rowbase, i0, (long long)p.l_q - i0, q_row_b, od, wave, lane_off);
    if (wave < 2) {
      // wave 0: LSE2 of the 64 rows, wave 1: D (rows past l_q read as 0)
      const float* src = (wave == 0 ? p.lse2 : p.dd) + ((size_t)b * p.h + hq) * p.l_q + i0;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(src), (short)0, (int)(4 * max(0, min(BQ, p.l_q - i0))), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(ld + wave * BQ), 4,
                                               (uint32_t)lane * 4u, 0, 0, 0);
    }
  };
  // masked scores become -inf * sign(c) (c is never 0), so that P = 0
  const float s_mask = p.c > 0.f ? kNegInf : -kNegInf;
  // P and dS of the previous tile (bf16 pairs): its dV/dK products run one
  // step late, beside the softmax of the current tile
  u32x4_t ppv[NPS], dspv[NPS];
  auto dvdk = [&](const unsigned char* ql, const unsigned char* ol) {
    uint32_t va = va0;
    asm volatile("" : "+v"(va));
#pragma unroll
    for (int t = 0; t < NPS; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(ol + t * 16 * RB + (va ^ (64u * db))));
        const s16x4_t dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(ol + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
        const u32x2_t d2 = __builtin_bit_cast(u32x2_t, dlo);
        const u32x2_t d3 = __builtin_bit_cast(u32x2_t, dhi);
        dvt[db] = mfma32x32x16(u32x4_t{d2[0], d2[1], d3[0], d3[1]}, ppv[t], dvt[db]);
        const s16x4_t qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(ql + t * 16 * RB + (va ^ (64u * db))));
        const s16x4_t qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(ql + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
        const u32x2_t q2 = __builtin_bit_cast(u32x2_t, qlo);
        const u32x2_t q3 = __builtin_bit_cast(u32x2_t, qhi);
        dkt[db] = mfma32x32x16(u32x4_t{q2[0], q2[1], q3[0], q3[1]}, dspv[t], dkt[db]);
      }
  };
  auto step = [&](auto first, int u, const unsigned char* ql, const unsigned char* ol,
                  const float* ll, const unsigned char* qp, const unsigned char* op,
                  unsigned char* qn, unsigned char* on, float* ln) {
    if (u + 1 < u_end) load(u + 1, qn, on, ln);
    const int i0 = (t_begin + u % nt) * BQ;
    const bool full = wave_live && (i0 + BQ <= p.l_q) && (kw + kKeysPerWave <= lk_) &&
                      ((long long)kw - (i0 + BQ - 1) >= dlo_) &&
                      ((long long)(kw + kKeysPerWave - 1) - i0 <= dhi_);
    uint32_t ka = ka0;
    asm volatile("" : "+v"(ka));
    // S = Q K^T and dP = dO V^T: [32 queries x 32 keys] blocks, lane = key.
    // The Q and dO operands are read from LDS AH1 product pairs ahead (with
    // one wave per SIMD nothing else covers the read latency), the query
    // blocks interleaved so that four accumulations are in flight.
    f32x16_t sa[NQB], dpa[NQB];
    {
      constexpr int AH1 = 3;
      constexpr int NX1 = NQB * NDS;
      u32x4_t ra[AH1 + 1], rb[AH1 + 1];
      auto rd1 = [&](int x) {
        const int s = x / NQB, qb = x % NQB;
        ra[x % (AH1 + 1)] =
            *reinterpret_cast<const u32x4_t*>(ql + qb * 32 * RB + (ka ^ (32u * s)));
        rb[x % (AH1 + 1)] =
            *reinterpret_cast<const u32x4_t*>(ol + qb * 32 * RB + (ka ^ (32u * s)));
      };
#pragma unroll
      for (int x = 0; x < AH1; ++x) rd1(x);
#pragma unroll
      for (int x = 0; x < NX1; ++x) {
        if (x + AH1 < NX1) rd1(x + AH1);
        const int s = x / NQB, qb = x % NQB;
        sa[qb] = mfma32x32x16(ra[x % (AH1 + 1)], kf[s], s == 0 ? f32x16_t{} : sa[qb]);
        dpa[qb] = mfma32x32x16(rb[x % (AH1 + 1)], vf[s], s == 0 ? f32x16_t{} : dpa[qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!full) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 32 * qb + 8 * (r >> 2) + 4 * half + (r & 3);
          const int rel = kj - i;
          const bool ok = (rel >= dlo_) & (rel <= dhi_) & (i < p.l_q) & (kj < lk_);
          sa[qb][r] = ok ? sa[qb][r] : s_mask;
        }
    }
    // P = exp2(c s - lse2), dS = P (dP - D); both packed to bf16.  Chunk
    // (qb, r4) gives the four k-slots 8 r4 + 4 half .. of query block qb.
    u32x4_t ppn[NPS], dsn[NPS];
    auto chunk = [&](int k) {
      const int qb = k / 4, r4 = k % 4;
      const int qi_loc = 32 * qb + 8 * r4 + 4 * half;
      const f32x4_t l2 = *reinterpret_cast<const f32x4_t*>(ll + qi_loc);
      const f32x4_t dv = *reinterpret_cast<const f32x4_t*>(ll + BQ + qi_loc);
      float pv[4], dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * r4 + e;
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sa[qb][r], p.c, -l2[e]));
        dsv[e] = pv[e] * (dpa[qb][r] - dv[e]);
      }
      const int t16 = 2 * qb + (r4 >> 1);
      const int w0 = (r4 & 1) * 2;
      ppn[t16][w0] = pack_bf16x2(pv[0], pv[1]);
      ppn[t16][w0 + 1] = pack_bf16x2(pv[2], pv[3]);
      dsn[t16][w0] = pack_bf16x2(dsv[0], dsv[1]);
      dsn[t16][w0 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      // pin the chunk here (keeps it from being sunk past the MFMAs it is
      // meant to run beside)
      asm volatile("" : "+v"(ppn[t16][w0]), "+v"(ppn[t16][w0 + 1]), "+v"(dsn[t16][w0]),
                   "+v"(dsn[t16][w0 + 1]));
    };
    constexpr int NK = 4 * NQB;  // chunks per tile
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int k = 0; k < NK; ++k) chunk(k);
    } else {
      // the previous tile's dV^T += dO^T P, dK^T += Q^T dS (pair x = t NDB +
      // db), operands read three pairs ahead, one softmax chunk per two pairs
      constexpr int NX = NPS * NDB;
      constexpr int AHEAD = 3;
      uint32_t va = va0;
      asm volatile("" : "+v"(va));
      s16x4_t opnd[AHEAD + 1][4];
      auto rd = [&](int x) {
        const int t = x / NDB, db = x % NDB;
        s16x4_t* o4 = opnd[x % (AHEAD + 1)];
        o4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(op + t * 16 * RB + (va ^ (64u * db))));
        o4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(op + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
        o4[2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(qp + t * 16 * RB + (va ^ (64u * db))));
        o4[3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(qp + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
      };
#pragma unroll
      for (int x = 0; x < AHEAD; ++x) rd(x);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        if (x + AHEAD < NX) rd(x + AHEAD);
        const int t = x / NDB, db = x % NDB;
        const s16x4_t* o4 = opnd[x % (AHEAD + 1)];
        const u32x2_t d2 = __builtin_bit_cast(u32x2_t, o4[0]);
        const u32x2_t d3 = __builtin_bit_cast(u32x2_t, o4[1]);
        const u32x2_t q2 = __builtin_bit_cast(u32x2_t, o4[2]);
        const u32x2_t q3 = __builtin_bit_cast(u32x2_t, o4[3]);
        dvt[db] = mfma32x32x16(u32x4_t{d2[0], d2[1], d3[0], d3[1]}, ppv[t], dvt[db]);
        dkt[db] = mfma32x32x16(u32x4_t{q2[0], q2[1], q3[0], q3[1]}, dspv[t], dkt[db]);
        // this tile's softmax chunks, spread evenly over the pairs
        const int k_lo = x * NK / NX, k_hi = (x + 1) * NK / NX;
#pragma unroll
        for (int k = k_lo; k < k_hi; ++k) chunk(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t = 0; t < NPS; ++t) {
      ppv[t] = ppn[t];
      dspv[t] = dsn[t];
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads landed
    __syncthreads();
  };
  const std::integral_constant<bool, true> kFirst;
  const std::integral_constant<bool, false> kLater;
  if (u_lo < u_end) {
    load(u_lo, q_lds0, o_lds0, l_lds0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    step(kFirst, u_lo, q_lds0, o_lds0, l_lds0, q_lds2, o_lds2, q_lds1, o_lds1, l_lds1);
  }
  // unrolled by three so that every buffer reference is a fixed LDS object
  for (int u = u_lo + 1; u < u_end; u += 3) {
    step(kLater, u, q_lds1, o_lds1, l_lds1, q_lds0, o_lds0, q_lds2, o_lds2, l_lds2);
    if (u + 1 < u_end)
      step(kLater, u + 1, q_lds2, o_lds2, l_lds2, q_lds1, o_lds1, q_lds0, o_lds0, l_lds0);
    if (u + 2 < u_end)
      step(kLater, u + 2, q_lds0, o_lds0, l_lds0, q_lds2, o_lds2, q_lds1, o_lds1, l_lds1);
  }
  if (u_lo < u_end) {
    // the last tile's dV/dK products, out of the buffer set it landed in
    const int r = (u_end - 1 - u_lo) % 3;
    if (r == 0) dvdk(q_lds0, o_lds0);
    else if (r == 1) dvdk(q_lds1, o_lds1);
    else dvdk(q_lds2, o_lds2);
    __syncthreads();
  }

  if (p.split > 1) {
    // ---- split: every slice stores its partial dK^T, dV^T (fp32, the
    // lane's key and dims 32 db + 8 r4 + 4 half + 0..3); bwd_dkdv_reduce
    // adds them up (slice 0 first) and writes dK, dV
    const size_t poff = ((size_t)b * lk_ + kj) * kv_row + (size_t)g * D + 4 * half;
    float* pk = p.part + (size_t)slice * 2 * p.part_half;
    if (kj <= last_key) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          *reinterpret_cast<f32x4_t*>(pk + poff + 32 * db + 8 * r4) =
              f32x4_t{dkt[db][4 * r4], dkt[db][4 * r4 + 1], dkt[db][4 * r4 + 2],
                      dkt[db][4 * r4 + 3]};
          *reinterpret_cast<f32x4_t*>(pk + p.part_half + poff + 32 * db + 8 * r4) =
              f32x4_t{dvt[db][4 * r4], dvt[db][4 * r4 + 1], dvt[db][4 * r4 + 2],
                      dvt[db][4 * r4 + 3]};
        }
    }
    return;
  }

  if constexpr (ACC) {
    // ---- epilogue (ACC): dk_acc += scale dK^T, dv_acc += dV^T in fp32; the
    // lane owns key kj and dims 32 db + 8 r4 + 4 half + 0..3 (16 bytes)
    if (kj <= last_key) {
      const size_t off = ((size_t)b * lk_ + kj) * kv_row + (size_t)g * D + 4 * half;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4_t* k4 = reinterpret_cast<f32x4_t*>(dka_ + off + 32 * db + 8 * r4);
          f32x4_t* v4 = reinterpret_cast<f32x4_t*>(dva_ + off + 32 * db + 8 * r4);
          const f32x4_t kx = {dkt[db][4 * r4], dkt[db][4 * r4 + 1], dkt[db][4 * r4 + 2],
                              dkt[db][4 * r4 + 3]};
          const f32x4_t vx = {dvt[db][4 * r4], dvt[db][4 * r4 + 1], dvt[db][4 * r4 + 2],
                              dvt[db][4 * r4 + 3]};
          *k4 = *k4 + kx * p.scale;
          *v4 = *v4 + vx;
        }
    }
    return;
  }
  // ---- epilogue: dK = scale dK^T, dV = dV^T as bf16, 32 key rows per wave
  // staged through LDS (dK rows in the Q buffers, dV rows in the dO buffers,
  // swizzled like the tiles) so that every store writes whole rows
  uint32_t ln = (uint32_t)lane;
  asm volatile("" : "+v"(ln));
  const uint32_t ecol = ln & 31u, ehalf = ln >> 5;
  unsigned char* stk = (wave < 2 ? q_lds0 : q_lds1) + (wave & 1) * 32 * RB;
  unsigned char* stv = (wave < 2 ? o_lds0 : o_lds1) + (wave & 1) * 32 * RB;
  static_assert(2 * 32 * RB <= TB, "staging fits");
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2_t wk, wv;
      wk[0] = pack_bf16x2(dkt[db][4 * r4] * p.scale, dkt[db][4 * r4 + 1] * p.scale);
      wk[1] = pack_bf16x2(dkt[db][4 * r4 + 2] * p.scale, dkt[db][4 * r4 + 3] * p.scale);
      wv[0] = pack_bf16x2(dvt[db][4 * r4], dvt[db][4 * r4 + 1]);
      wv[1] = pack_bf16x2(dvt[db][4 * r4 + 2], dvt[db][4 * r4 + 3]);
      const uint32_t c = (uint32_t)(4 * db + r4) ^ chunk_swz<D>(ecol);
      *reinterpret_cast<u32x2_t*>(stk + ecol * RB + c * 16 + 8 * ehalf) = wk;
      *reinterpret_cast<u32x2_t*>(stv + ecol * RB + c * 16 + 8 * ehalf) = wv;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int x = 0; x < 32 / RPI; ++x) {
    const int r = x * RPI + (int)(ln / CPR);
    const uint32_t c = (ln % CPR) ^ chunk_swz<D>((uint32_t)r);
    const u32x4_t vk = *reinterpret_cast<const u32x4_t*>(stk + r * RB + c * 16);
    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(stv + r * RB + c * 16);
    if (kw + r <= last_key) {
      const size_t off = ((size_t)b * lk_ + kw + r) * kv_row + (size_t)g * D + 8 * (ln % CPR);
      *reinterpret_cast<u32x4_t*>(p.dk + off) = vk;
      *reinterpret_cast<u32x4_t*>(p.dv + off) = vv;
    }
  }
}

// Sum of the split dK/dV partials, slice 0 first (the order does not depend
// on scheduling, so results are bitwise repeatable), then the epilogue: dK =
// scale sum, dV = sum, written as bf16 or (ACC) added to the fp32
// accumulators.  Four elements per thread, consecutive in memory.
template <bool ACC>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_reduce(BwdParams p) {
  const long long n4 = (long long)(p.part_half / 4);
  const long long e = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n4) return;
  f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < p.split; ++sl) {
    const float* pk = p.part + (size_t)sl * 2 * p.part_half;
    sk = sk + reinterpret_cast<const f32x4_t*>(pk)[e];
    sv = sv + reinterpret_cast<const f32x4_t*>(pk + p.part_half)[e];
  }
  sk = sk * p.scale;
  if constexpr (ACC) {
    f32x4_t* dk = reinterpret_cast<f32x4_t*>(p.dk_acc) + e;
    f32x4_t* dv = reinterpret_cast<f32x4_t*>(p.dv_acc) + e;
    *dk = *dk + sk;
    *dv = *dv + sv;
  } else {
    u32x2_t wk, wv;
    wk[0] = pack_bf16x2(sk[0], sk[1]);
    wk[1] = pack_bf16x2(sk[2], sk[3]);
    wv[0] = pack_bf16x2(sv[0], sv[1]);
    wv[1] = pack_bf16x2(sv[2], sv[3]);
    reinterpret_cast<u32x2_t*>(p.dk)[e] = wk;
    reinterpret_cast<u32x2_t*>(p.dv)[e] = wv;
  }
}

// ------------------------------------------------------------ dQ
//
// One workgroup per 128 query rows of one head, 4 waves x 32 rows; the
// wave's Q and dO rows stay in VGPRs as B operands, its LSE and D per lane.
// Key tiles of 64 rows of K and V stream through LDS (swizzled rows, two
// buffers, one tile ahead, direct buffer loads).  Per tile: S^T = K Q^T and
// dP^T = V dO^T (K and V rows as A operands) put one query per lane;
// P^T = exp2(c S^T - LSE2), dS^T = P^T (dP^T - D), and dQ^T += K^T dS^T with
// K^T read transposed out of the row-major K tile reads dS^T straight from
// registers as its B operand.
//
// KSPLIT = 2: eight waves in two groups of four over the same 128 rows, each
// group with its own LDS buffers and alternate key tiles; dQ is a plain sum
// over keys, so group 1's partial dQ^T is simply added to group 0's (through
// LDS) before the epilogue.
//
// WIDE: eight waves over 256 rows, one group: every K/V tile loaded once
// for twice the rows.

template <int D, bool ACC, int KSPLIT, bool MULTI, bool WIDE = false>
__global__ __launch_bounds__(kThreads * (WIDE ? 2 : KSPLIT), KSPLIT == 1 && !WIDE ? 2 : 1)
    void bwd_dq_kernel(BwdParams p, int n_qtiles, int reverse) {
  static_assert(!MULTI || !ACC, "the multi-chunk form writes dQ");
  static_assert(!WIDE || (KSPLIT == 1 && !MULTI), "wide: one group of eight waves");
  constexpr int BN = 64;
  constexpr int RB = D * 2;
  constexpr int TB = BN * RB;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  constexpr int NPS = BN / 16;
  // WIDE: eight waves over 256 rows share every K/V tile (half the tile
  // loads per product of four waves over 128 rows)
  constexpr int BM = WIDE ? 256 : 128;
  constexpr uint32_t kVC = D == 128 ? 32u : 16u;
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[KSPLIT][TB];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds1[KSPLIT][TB];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[KSPLIT][TB];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds1[KSPLIT][TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = KSPLIT == 1 ? 0 : wave_all / 4;         // key group
  const int wave = KSPLIT == 1 ? wave_all : wave_all % 4;  // query block of this wave
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
  const uint32_t kv_row_b = (uint32_t)kv_row * 2u;
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

  // MULTI: the key tiles of every chunk in turn, each with its own tensors,
  // length and mask bounds, one dQ^T accumulation over all of them
  const int n_ch = MULTI ? p.n_chunks : 1;
  for (int ci = 0; ci < n_ch; ++ci) {
  // the chunk's key side (locals: p is never written, see bwd_dkdv_kernel)
  const uint16_t* kp_ = MULTI ? p.ch[ci].k : p.k;
  const uint16_t* vp_ = MULTI ? p.ch[ci].v : p.v;
  const int lk_ = MULTI ? p.ch[ci].l_k : p.l_k;
  const int dlo_ = MULTI ? p.ch[ci].dlo : p.dlo;
  const int dhi_ = MULTI ? p.ch[ci].dhi : p.dhi;
  const long long jlo = max(0LL, (long long)i0 + dlo_);
  const long long jhi = min((long long)lk_ - 1,
                            (long long)min(i0 + BM - 1, last_row) + dhi_);
  const int wa = iw;
  const int wb = min(iw + 31, last_row);
  const bool wave_live = wa <= last_row;
  const long long wjlo = max(0LL, (long long)wa + dlo_);
  const long long wjhi = min((long long)lk_ - 1, (long long)wb + dhi_);
  const uint16_t* kbase = kp_ + (size_t)b * lk_ * kv_row + (size_t)g * D;
  const uint16_t* vbase = vp_ + (size_t)b * lk_ * kv_row + (size_t)g * D;

  const uint32_t lane_off = tile_lane_offset<D>(wave, lane, kv_row_b);
  uint32_t ka0, va0;
  lds_read_bases<D>(lane, ka0, va0);
  // this wave's share of the loads of one 64-key tile (WIDE: one of eight
  // waves, rows (8 x + wave) RPL + lane / CPR of load x)
  auto dma_tile = [&](const uint16_t* base, long long j0, unsigned char* dst) {
    if constexpr (!WIDE) {
      tile_dma<D>(base, j0, (long long)lk_ - j0, kv_row_b, dst, wave, lane_off);
    } else {
      constexpr int RPL = 1024 / RB;
      constexpr int LOADS = BN / RPL / 8;
      static_assert(LOADS >= 1 && (8 * RPL) % 16 == 0, "wide tile loads");
      const long long bytes =
          max(0LL, min(((long long)lk_ - j0) * (long long)kv_row_b, 0x7fffffffLL));
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base) + (size_t)j0 * (kv_row_b / 2), (short)0, (int)bytes,
          0x00020000);
#pragma unroll
      for (int x = 0; x < LOADS; ++x) {
        const int row0 = (x * 8 + wave) * RPL;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + row0 * RB), 16,
                                                 lane_off,
                                                 (uint32_t)(x * 8 * RPL) * kv_row_b, 0, 0);
      }
    }
  };
  auto load = [&](int kt, unsigned char* kd, unsigned char* vd) {
    const long long j0 = (long long)kt * BN;
    dma_tile(kbase, j0, kd);
    dma_tile(vbase, j0, vd);
  };

  int kt_begin = 0, kt_end = 0;
  if (jlo <= jhi) {
    kt_begin = (int)(jlo / BN);
    kt_end = (int)(jhi / BN) + 1;
  }
  const float s_mask = p.c > 0.f ? kNegInf : -kNegInf;
  auto step = [&](int kt, const unsigned char* kl, const unsigned char* vl, unsigned char* kn,
                  unsigned char* vn) {
    if (kt + KSPLIT < kt_end) load(kt + KSPLIT, kn, vn);
    const int j0 = kt * BN;
    const bool live = wave_live && (long long)j0 <= wjhi && (long long)(j0 + BN - 1) >= wjlo;
    if (live) {
      const bool full = (j0 + BN <= lk_) && ((long long)j0 - wb >= dlo_) &&
                        ((long long)(j0 + BN - 1) - wa <= dhi_);
      uint32_t ka = ka0, va = va0;
      asm volatile("" : "+v"(ka), "+v"(va));
      // S^T = K Q^T and dP^T = V dO^T: lane = query
      f32x16_t sa[NKB], dpa[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kl + kb * 32 * RB + (ka ^ (32u * s)));
          sa[kb] = mfma32x32x16(a, qf[s], s == 0 ? f32x16_t{} : sa[kb]);
          const u32x4_t a2 = *reinterpret_cast<const u32x4_t*>(vl + kb * 32 * RB + (ka ^ (32u * s)));
          dpa[kb] = mfma32x32x16(a2, dof[s], s == 0 ? f32x16_t{} : dpa[kb]);
        }
      // masked scores become -inf * sign(c) (c is never 0), so that P = 0;
      // masking the scores rather than P keeps the exponentials unconditional
      // (masking P made the compiler put every exponential under a branch)
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            const int rel = j - qi;
            const bool ok = (rel >= dlo_) & (rel <= dhi_) & (j < lk_);
            sa[kb][r] = ok ? sa[kb][r] : s_mask;
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
            const float pe = __builtin_amdgcn_exp2f(fmaf(sa[kb][r + e], p.c, -l2));
            ds2[e] = pe * (dpa[kb][r + e] - dval);
          }
          dsp[2 * kb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(ds2[0], ds2[1]);
        }
      // dQ^T += K^T dS^T   (k-slots = keys)
#pragma unroll
      for (int t = 0; t < NPS; ++t)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_ptr)(kl + t * 16 * RB + (va ^ (64u * db))));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_ptr)(kl + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
          const u32x2_t l2v = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t h2v = __builtin_bit_cast(u32x2_t, hi);
          dqt[db] = mfma32x32x16(u32x4_t{l2v[0], l2v[1], h2v[0], h2v[1]}, dsp[t], dqt[db]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads landed
    __syncthreads();
  };
  // this group's key tiles: kt_begin + grp + KSPLIT u; both groups run the
  // same number of steps (and barriers), idling past their last tile
  const int kt_first = kt_begin + grp;
  const int n_steps = (kt_end - kt_begin + KSPLIT - 1) / KSPLIT;
  if (kt_begin < kt_end) {
    if (kt_first < kt_end) load(kt_first, k_lds0[grp], v_lds0[grp]);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }
  // unrolled by two so that every buffer reference is a fixed LDS object
  if constexpr (KSPLIT == 1) {
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      step(kt, k_lds0[0], v_lds0[0], k_lds1[0], v_lds1[0]);
      if (kt + 1 < kt_end) step(kt + 1, k_lds1[0], v_lds1[0], k_lds0[0], v_lds0[0]);
    }
  } else {
    for (int u = 0; u < n_steps; u += 2) {
      const int kt = kt_first + KSPLIT * u;
      if (kt < kt_end) step(kt, k_lds0[grp], v_lds0[grp], k_lds1[grp], v_lds1[grp]);
      else __syncthreads();
      if (u + 1 < n_steps) {
        if (kt + KSPLIT < kt_end)
          step(kt + KSPLIT, k_lds1[grp], v_lds1[grp], k_lds0[grp], v_lds0[grp]);
        else __syncthreads();
      }
    }
  }
  }  // chunks
  if constexpr (KSPLIT == 2) {
    // ---- add group 1's partial dQ^T to group 0's through LDS (float4 f =
    // 4 db + r4 of lane wl at (f, wl), spread over the two V buffers)
    const int wl = wave * 64 + lane;
    float4* xo0 = reinterpret_cast<float4*>(&v_lds0[0][0]);
    float4* xo1 = reinterpret_cast<float4*>(&v_lds1[0][0]);
    static_assert(NDB * 2 * kThreads * 16 <= KSPLIT * TB, "exchange fits");
    if (grp == 1) {
#pragma unroll
      for (int f = 0; f < 4 * NDB; ++f)
        (f < 2 * NDB ? xo0 : xo1)[(f % (2 * NDB)) * kThreads + wl] =
            make_float4(dqt[f / 4][4 * (f % 4)], dqt[f / 4][4 * (f % 4) + 1],
                        dqt[f / 4][4 * (f % 4) + 2], dqt[f / 4][4 * (f % 4) + 3]);
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int f = 0; f < 4 * NDB; ++f) {
      const float4 x = (f < 2 * NDB ? xo0 : xo1)[(f % (2 * NDB)) * kThreads + wl];
      dqt[f / 4][4 * (f % 4)] += x.x;
      dqt[f / 4][4 * (f % 4) + 1] += x.y;
      dqt[f / 4][4 * (f % 4) + 2] += x.z;
      dqt[f / 4][4 * (f % 4) + 3] += x.w;
    }
  }

  if constexpr (ACC) {
    // ---- epilogue (ACC): dq_acc += scale dQ^T in fp32; the lane owns query
    // row qi and dims 32 db + 8 r4 + 4 half + 0..3 (16 bytes)
    if (qi <= last_row) {
      const size_t off = ((size_t)b * p.l_q + qi) * q_row + (size_t)hq * D + 4 * half;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4_t* q4 = reinterpret_cast<f32x4_t*>(p.dq_acc + off + 32 * db + 8 * r4);
          const f32x4_t x = {dqt[db][4 * r4], dqt[db][4 * r4 + 1], dqt[db][4 * r4 + 2],
                             dqt[db][4 * r4 + 3]};
          *q4 = *q4 + x * p.scale;
        }
    }
    return;
  }
  // ---- epilogue: dQ = scale dQ^T as bf16, the wave's 32 rows staged
  // through LDS (swizzled like the tiles) so that every store writes whole
  // rows
  uint32_t ln = (uint32_t)lane;
  asm volatile("" : "+v"(ln));
  const uint32_t ecol = ln & 31u, ehalf = ln >> 5;
  const int w2 = wave >> 1;   // two waves to each buffer (WIDE: all four)
  unsigned char* stage = (w2 == 0 ? &k_lds0[0][0] : w2 == 1 ? &k_lds1[0][0]
                          : w2 == 2 ? &v_lds0[0][0] : &v_lds1[0][0]) + (wave & 1) * 32 * RB;
  static_assert(2 * 32 * RB <= TB, "staging fits");
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2_t w;
      w[0] = pack_bf16x2(dqt[db][4 * r4] * p.scale, dqt[db][4 * r4 + 1] * p.scale);
      w[1] = pack_bf16x2(dqt[db][4 * r4 + 2] * p.scale, dqt[db][4 * r4 + 3] * p.scale);
      const uint32_t c = (uint32_t)(4 * db + r4) ^ chunk_swz<D>(ecol);
      *reinterpret_cast<u32x2_t*>(stage + ecol * RB + c * 16 + 8 * ehalf) = w;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int x = 0; x < 32 / RPI; ++x) {
    const int r = x * RPI + (int)(ln / CPR);
    const uint32_t c = (ln % CPR) ^ chunk_swz<D>((uint32_t)r);
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stage + r * RB + c * 16);
    if (iw + r <= last_row)
      *reinterpret_cast<u32x4_t*>(p.dq + ((size_t)b * p.l_q + iw + r) * q_row +
                                  (size_t)hq * D + 8 * (ln % CPR)) = val;
  }
}

// dK/dV workgroups per (key tile, key/value head) pair: when the key tiles
// alone give fewer than two workgroups per CU, the query steps of each key
// tile are split over up to four workgroups, whose partial sums a second
// kernel adds up in a fixed order.
constexpr int kDkdvTargetWGs = 512;
constexpr int kDqCUs = 256;

int dkdv_split(int n, int l_k, int h_kv) {
  const long long w = (long long)((l_k + kKeysPerWG - 1) / kKeysPerWG) * n * h_kv;
  if (w >= kDkdvTargetWGs) return 1;
  return (int)std::min<long long>(4, (kDkdvTargetWGs + w - 1) / w);
}

// Workspace layout: D and LSE2 per query row, then (split > 1) the per-slice
// dK, dV partials, each part 256-byte aligned.
struct BwdWorkspace {
  size_t dd, lse2, part, total;
  size_t part_half;  // floats in one partial dK (or dV)
  int split;
};

BwdWorkspace bwd_layout(int n, int l_q, int l_k, int h, int h_kv, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdWorkspace w;
  const size_t rows = (size_t)n * l_q * h;
  w.split = dkdv_split(n, l_k, h_kv);
  w.part_half = w.split > 1 ? (size_t)n * l_k * h_kv * d : 0;
  w.dd = 0;
  w.lse2 = up(rows * 4);
  w.part = w.lse2 + up(rows * 4);
  w.total = w.part + up((size_t)w.split * 2 * w.part_half * 4);
  return w;
}

template <int D>
void launch_pre_d(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.n * p.l_q * p.h;
  const long long pre_blocks = (rows * (D / 8) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(capped_grid(pre_blocks)), dim3(kThreads),
                     0, stream, p);
}

template <int D, bool ACC>
hipError_t launch_bwd_d(const BwdParams& p, int causal, hipStream_t stream, bool prepared) {
  if (!prepared) launch_pre_d<D>(p, stream);
  const int n_ktiles = (p.l_k + kKeysPerWG - 1) / kKeysPerWG;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, ACC, false>),
                     dim3((unsigned)(p.split * n_ktiles * p.n * p.h_kv)), dim3(kThreads),
                     0, stream, p, n_ktiles, causal ? 1 : 0);
  if (p.split > 1) {
    const long long n4 = (long long)(p.part_half / 4);
    hipLaunchKernelGGL((bwd_dkdv_reduce<ACC>), dim3((unsigned)((n4 + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, p);
  }
  // dQ: with fewer than two workgroups per CU, each workgroup's key tiles
  // are split over two groups of four waves that add their partial dQ at
  // the end; at d = 128 with at least one 256-row workgroup per CU, eight
  // waves share each tile (two waves per SIMD in every form; at d = 64 the
  // four-wave form runs three per SIMD)
  const int n_qtiles = (p.l_q + 127) / 128;
  const long long dq_wgs = (long long)n_qtiles * p.n * p.h;
  const int n_wide = (p.l_q + 255) / 256;
  const long long wide_wgs = (long long)n_wide * p.n * p.h;
  if (dq_wgs < 2 * kDqCUs) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, ACC, 2, false>), dim3((unsigned)dq_wgs), dim3(2 * kThreads),
                       0, stream, p, n_qtiles, causal ? 1 : 0);
    return hipGetLastError();
  }
  if constexpr (D == 128) {
    if (wide_wgs >= kDqCUs) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, ACC, 1, false, true>), dim3((unsigned)wide_wgs),
                         dim3(2 * kThreads), 0, stream, p, n_wide, causal ? 1 : 0);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, ACC, 1, false>), dim3((unsigned)dq_wgs), dim3(kThreads),
                     0, stream, p, n_qtiles, causal ? 1 : 0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_ring_d(const BwdParams& p, int total_wgs, int causal,
                             hipStream_t stream) {
  launch_pre_d<D>(p, stream);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true>), dim3((unsigned)total_wgs),
                     dim3(kThreads), 0, stream, p, 0, causal ? 1 : 0);
  const int n_qtiles = (p.l_q + 127) / 128;
  const long long dq_wgs = (long long)n_qtiles * p.n * p.h;
  if (dq_wgs < 2 * kDqCUs)
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, 2, true>), dim3((unsigned)dq_wgs),
                       dim3(2 * kThreads), 0, stream, p, n_qtiles, causal ? 1 : 0);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, 1, true>), dim3((unsigned)dq_wgs),
                       dim3(kThreads), 0, stream, p, n_qtiles, causal ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_ring(const void* dout, const void* q, const void* out, const float* lse,
                           const BwdChunkArgs* chunks, int n_chunks, void* dq,
                           const AttnShape& s, void* workspace, hipStream_t stream) {
  BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  const BwdWorkspace w = bwd_layout(s.n, s.l_q, 1, s.h, 1, s.d);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  p.dd = reinterpret_cast<float*>(ws + w.dd);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.split = 1;
  p.n = s.n;
  p.l_q = s.l_q;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  p.c = s.scale == 0.f ? 1e-30f : s.scale * kLog2e;
  p.scale = s.scale;
  p.n_chunks = n_chunks;
  int wgs = 0;
  for (int c = 0; c < n_chunks; ++c) {
    BwdChunk& ch = p.ch[c];
    ch.k = static_cast<const uint16_t*>(chunks[c].k);
    ch.v = static_cast<const uint16_t*>(chunks[c].v);
    ch.dk_acc = chunks[c].dk_acc;
    ch.dv_acc = chunks[c].dv_acc;
    ch.l_k = chunks[c].l_k;
    ch.dlo = chunks[c].dlo;
    ch.dhi = chunks[c].dhi;
    ch.ktiles = (chunks[c].l_k + kKeysPerWG - 1) / kKeysPerWG;
    ch.wg_begin = wgs;
    wgs += ch.ktiles * s.n * s.h_kv;
  }
  // the single-chunk fields hold the first chunk (read only where the
  // multi-chunk kernels have replaced them)
  p.k = p.ch[0].k;
  p.v = p.ch[0].v;
  p.l_k = p.ch[0].l_k;
  p.dlo = p.ch[0].dlo;
  p.dhi = p.ch[0].dhi;
  return s.d == 128 ? launch_bwd_ring_d<128>(p, wgs, s.causal, stream)
                    : launch_bwd_ring_d<64>(p, wgs, s.causal, stream);
}

size_t bwd_workspace_bytes(int n, int l_q, int l_k, int h, int h_kv, int d) {
  return bwd_layout(n, l_q, l_k, h, h_kv, d).total;
}

size_t bwd_prepared_bytes(int n, int l_q, int h) {
  // D and LSE2 come first in every layout, whatever the key count
  return bwd_layout(n, l_q, 1, h, 1, 64).part;
}

void bwd_prepared_rows(void* workspace, int n, int l_q, int h, float** dd, float** lse2) {
  const BwdWorkspace w = bwd_layout(n, l_q, 1, h, 1, 64);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  *dd = reinterpret_cast<float*>(ws + w.dd);
  *lse2 = reinterpret_cast<float*>(ws + w.lse2);
}

hipError_t launch_bwd_prepare(const void* dout, const void* out, const float* lse, int n,
                              int l_q, int h, int d, void* workspace, hipStream_t stream) {
  BwdParams p{};
  p.dout = static_cast<const uint16_t*>(dout);
  p.o = static_cast<const uint16_t*>(out);
  p.lse = lse;
  const BwdWorkspace w = bwd_layout(n, l_q, 1, h, 1, d);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  p.dd = reinterpret_cast<float*>(ws + w.dd);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.n = n;
  p.l_q = l_q;
  p.h = h;
  if (d == 128) launch_pre_d<128>(p, stream);
  else launch_pre_d<64>(p, stream);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* dout, const void* q, const void* k,
                      const void* v, const void* out, const float* lse,
                      void* dq, void* dk, void* dv, const AttnShape& s,
                      void* workspace, bool bf16, hipStream_t stream,
                      float* dq_acc, float* dk_acc, float* dv_acc, bool prepared) {
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
  p.dq_acc = dq_acc;
  p.dk_acc = dk_acc;
  p.dv_acc = dv_acc;
  const BwdWorkspace w = bwd_layout(s.n, s.l_q, s.l_k, s.h, s.h_kv, s.d);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  p.dd = reinterpret_cast<float*>(ws + w.dd);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.part = reinterpret_cast<float*>(ws + w.part);
  p.part_half = w.part_half;
  p.split = w.split;
  p.n = s.n;
  p.l_q = s.l_q;
  p.l_k = s.l_k;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  // never 0: a masked score then always gives c s = -inf (P is unchanged)
  p.c = s.scale == 0.f ? 1e-30f : s.scale * kLog2e;
  p.scale = s.scale;
  p.dlo = s.dlo;
  p.dhi = s.dhi;
  if (dq_acc != nullptr)
    return s.d == 128 ? launch_bwd_d<128, true>(p, s.causal, stream, prepared)
                      : launch_bwd_d<64, true>(p, s.causal, stream, prepared);
  return s.d == 128 ? launch_bwd_d<128, false>(p, s.causal, stream, prepared)
                    : launch_bwd_d<64, false>(p, s.causal, stream, prepared);
}

}  // namespace bea
