// Exact attention forward for gfx950: blockwise over key tiles with an online
// softmax, bf16 MFMA with fp32 accumulation (and an fp32 SIMT variant).
//
// What is computed follows the pages "picotron/parallel/context_parallel.py"
// (ring_attention_forward: S = scale * Q K^T, causal mask, LSE = log sum exp,
// O = softmax(S) V; RingAttention._repeat_kv for grouped heads) and
// "flash_sharding.py" (ring_fwd: the (O, LSE) pair per query row, a row with
// no allowed key gives O = 0 and LSE = -inf; the log1p merge, which the
// online softmax applies per key tile).
//
// bf16 kernel layout (one key group = 4 waves = 128 query rows of one head;
// a workgroup holds one key group, or two that split the key tiles, see
// KSPLIT below):
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the
//    A operand, the wave's Q rows stay in VGPRs as the B operand for the whole
//    key loop.  In the result every lane holds one query (lane % 32) and 16
//    keys per 32-key block, so a row max needs one cross-half exchange and a
//    row sum none until the epilogue.
//  * O^T = V^T P^T reuses the S^T registers directly as the B operand (the
//    contraction order over keys is free, so the 8 keys a lane holds become
//    the 8 k-slots it supplies).  The matching A operand (8 keys of one dim)
//    comes from the row-major V tile through two transposing LDS reads.
//  * K and V tiles of 64 keys are double-buffered in LDS and filled by
//    direct global-to-LDS buffer loads one tile ahead; one barrier per tile.
//  * Key tiles wholly outside a workgroup's causal/window band are never
//    visited; tiles wholly inside run without per-element mask work.
//  * The normalised O rows leave through LDS, so that each global store
//    writes whole rows rather than 16-byte pieces of 32 rows.
//  * The ACC instantiations (one fused ring step) merge (O, LSE) into a
//    float32 accumulator in the epilogue instead of writing them.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace bea {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kThreads = 64 * kWaves;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* acc;      // ACC kernels: fp32 accumulator O [n, l_q, h, d] (else unused)
  float* lse_acc;  // ACC kernels: its LSE [n, h, l_q] (natural log)
  int l_q, l_k, h, h_kv, grp;
  int n_heads;     // n * h
  int n_qtiles;
  int n_units;     // workgroups per head: n_qtiles, or ceil(n_qtiles / 2) paired
  int pairs;       // 1: workgroup r takes q tiles n_qtiles-1-r and r
  int xcd_groups;  // 1: keep the workgroups of one key/value head on one XCD
  int reverse;     // 1: launch the last (longest, under causal) q tiles first
  float c;         // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t q_and;  // Q fragment mask: 0 when scale == 0
  uint32_t q_xor;  // Q sign flip: 0x80008000 when scale < 0
  int dlo, dhi;
};

// blockIdx.x -> (work unit, flattened head b*h + hq); a unit is one q tile,
// or under pairing the two q tiles n_qtiles-1-r and r, whose key counts add up
// to about the same total for every r under a causal mask.
//
// Workgroups are handed to the 8 XCDs round-robin by id, and each XCD has its
// own L2.  When the key/value groups split evenly over the XCDs, every
// workgroup that reads one key/value head is given an id of the same residue
// mod 8, so that head's K/V tiles are fetched into one L2 only.  Under causal
// masking the last q tiles see the most keys; they get the lowest ids.
__device__ __forceinline__ void map_block(const FwdParams& p, int& unit,
                                          int& head) {
  const int w = blockIdx.x;
  int rank;
  if (p.xcd_groups) {
    const int xcd = w & 7;
    const int slot = w >> 3;
    const int per_xcd = p.n_heads >> 3;
    rank = slot / per_xcd;
    const int rem = slot - rank * per_xcd;
    const int gi = rem / p.grp;
    const int in_group = rem - gi * p.grp;
    head = (xcd + 8 * gi) * p.grp + in_group;
  } else {
    rank = w / p.n_heads;
    head = w - rank * p.n_heads;
  }
  unit = p.reverse ? (p.n_units - 1 - rank) : rank;
}

// The other half-wave's copy of x (lane l <-> lane l ^ 32), then combined:
// v_permlane32_swap hands lanes 0-31 the upper half's value in its second
// result and lanes 32-63 the lower half's value in its first result, so
// max/sum of the two results is the max/sum over the pair on every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Growth of the running row max (log2 units) that forces a rescale of the
// accumulators.  Below it the stale max is kept: exponentials are then at most
// 2^8, exact in meaning (O = sum p v / sum p for any fixed shift) and far from
// fp32 or bf16 range limits.
constexpr float kRescaleSlack = 8.f;

// KSPLIT = 2: eight waves per workgroup in two groups of four that cover the
// same 128 query rows and take alternate key tiles, each group with its own
// LDS buffers and online-softmax state; the two partial rows are merged at
// the end like two ring chunks.  A q tile then finishes in about half the
// time with one workgroup per CU, which lets a small or causal-imbalanced
// grid run longest-first and balance.  Under pairing a workgroup takes two q
// tiles one after the other (the short and the long one of a causal pair).
//
// ACC: instead of writing O and LSE, merge them into the fp32 accumulator
// (acc, lse_acc) in the epilogue, as one ring step followed by attn_merge
// would, without the block's O passing through HBM in bf16.
template <int D, int BN, int KSPLIT, bool ACC>
__global__ __launch_bounds__(kThreads * KSPLIT, KSPLIT == 1 ? 2 : 1) void fwd_bf16_kernel(
    FwdParams p) {
  static_assert(BN == 64, "tile of 64 keys");
  constexpr int RB = D * 2;          // bytes per tile row
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int ROWS_PER_DMA = 1024 / RB;  // rows one wave-wide DMA writes
  constexpr int DMA_PER_WAVE = BN / ROWS_PER_DMA / kWaves;
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDS = D / 16;    // 16-wide dim slices (S^T MFMA k steps)
  constexpr int NDB = D / 32;    // 32-dim blocks of O^T
  constexpr int NPS = BN / 16;   // 16-key slices (O^T MFMA k steps)
  constexpr uint32_t kVC = D == 128 ? 32u : 16u;   // chunk-bit flip of read c = 1

  // four separate LDS objects (one slot per key group in each), so the
  // compiler can tell the buffer being read from the one the DMA is filling
  // and need not wait for the DMA
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[KSPLIT][BN * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds1[KSPLIT][BN * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[KSPLIT][BN * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds1[KSPLIT][BN * D * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave: keep it (and the band and
  // tile bookkeeping derived from it) in scalar registers
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / kWaves;   // key group (0 unless KSPLIT = 2)
  const int wave = wave_all % kWaves;  // query block of this wave
  const int half = lane >> 5;
  const int col = lane & 31;

  // one q tile: the whole key loop, the merge of the key groups and the
  // epilogue
  auto fwd_tile = [&](const int tile, const int head) {
    const int b = head / p.h;
    const int hq = head - b * p.h;
    const int g = hq / p.grp;

    const int last_row = p.l_q - 1;
    const int i0 = tile * kBM;
    const int iw = i0 + wave * 32;
    const int qi = iw + col;

    // Key-tile range of the workgroup (rows i0 .. min(i0+kBM, l_q)-1).
    const long long jlo = max(0LL, (long long)i0 + p.dlo);
    const long long jhi = min((long long)p.l_k - 1,
                              (long long)min(i0 + kBM - 1, last_row) + p.dhi);
    int kt_begin = 0, kt_end = 0;
    if (jlo <= jhi) {
      kt_begin = (int)(jlo / BN);
      kt_end = (int)(jhi / BN) + 1;
    }
    // Key range of this wave.
    const int wa = iw;
    const int wb = min(iw + 31, last_row);
    const bool wave_live = wa <= last_row;
    const long long wjlo = max(0LL, (long long)wa + p.dlo);
    const long long wjhi = min((long long)p.l_k - 1, (long long)wb + p.dhi);

    // Q fragment: B operand of S^T = K Q^T, resident for the whole loop.  The
    // sign of the scale is folded into Q (sign-bit flip, exact) and a zero
    // scale becomes Q = 0 with c = log2(e) (every allowed score is then 0, as
    // scale * q.k is), so c > 0 below and a masked score of -inf always gives
    // exp2(-inf) = 0.
    const size_t q_row = (size_t)p.h * D;
    const uint16_t* qptr = p.q + ((size_t)b * p.l_q + min(qi, last_row)) * q_row +
                           (size_t)hq * D + 8 * half;
    u32x4_t qf[NDS];
  #pragma unroll
    for (int s = 0; s < NDS; ++s)
      qf[s] = (*reinterpret_cast<const u32x4_t*>(qptr + 16 * s) & p.q_and) ^ p.q_xor;

    f32x16_t oacc[NDB];
  #pragma unroll
    for (int db = 0; db < NDB; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = kNegInf;  // row max used for the exponentials (log2 units)
    float lsum = 0.f;   // this lane's half of the running row sum

    const size_t kv_row = (size_t)p.h_kv * D;
    const uint16_t* kbase = p.k + (size_t)b * p.l_k * kv_row + (size_t)g * D;
    const uint16_t* vbase = p.v + (size_t)b * p.l_k * kv_row + (size_t)g * D;
    const uint32_t kv_row_b = (uint32_t)kv_row * 2u;

    // DMA: instruction x of wave w writes rows (kWaves x + w) ROWS_PER_DMA + ...;
    // each lane fetches the logical chunk the swizzle places at its slot.
    const uint32_t dma_row = (uint32_t)(wave * ROWS_PER_DMA + lane / CPR);
    const uint32_t dma_off =
        dma_row * kv_row_b + (((uint32_t)(lane % CPR)) ^ chunk_swz<D>(dma_row)) * 16u;
    auto dma_tile = [&](const uint16_t* base, unsigned char* lds, int kt) {
      const long long rows = (long long)p.l_k - (long long)kt * BN;
      const long long bytes = min(rows * (long long)kv_row_b, 0x7fffffffLL);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base + (size_t)kt * BN * kv_row), (short)0, (int)bytes,
          0x00020000);
  #pragma unroll
      for (int x = 0; x < DMA_PER_WAVE; ++x) {
        const int row0 = (x * kWaves + wave) * ROWS_PER_DMA;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void_ptr)(lds + row0 * RB), 16, dma_off,
            (uint32_t)(x * kWaves * ROWS_PER_DMA) * kv_row_b, 0, 0);
      }
    };
    auto load_tile = [&](int kt, unsigned char* kd, unsigned char* vd) {
      dma_tile(kbase, kd, kt);
      dma_tile(vbase, vd, kt);
    };

    uint32_t ka0, va0;
    lds_read_bases<D>(lane, ka0, va0);

    auto live = [&](int kt) {
      const long long j0 = (long long)kt * BN;
      return wave_live && j0 <= wjhi && j0 + BN - 1 >= wjlo;
    };

    // One tile: S^T = K Q^T, mask (boundary tiles), online softmax, O += P V,
    // reading buffers (kl, vl).  The DMA of this group's next tile into the
    // other buffers (last read one step earlier) is in flight meanwhile; the
    // barrier at the end publishes it.
    auto step = [&](int kt, const unsigned char* kl, const unsigned char* vl,
                    unsigned char* kn, unsigned char* vn) {
      if (kt + KSPLIT < kt_end) load_tile(kt + KSPLIT, kn, vn);
      if (live(kt)) {
        // the empty asm keeps the derived addresses from being hoisted and
        // held live across the loop
        uint32_t ka = ka0, va = va0;
        asm volatile("" : "+v"(ka), "+v"(va));
        f32x16_t sacc[NKB];
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
  #pragma unroll
          for (int s = 0; s < NDS; ++s) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                kl + kb * 32 * RB + (ka ^ (32u * s)));
            sacc[kb] = mfma32x32x16(a, qf[s], sacc[kb]);
          }
        }
        const int j0 = kt * BN;
        const bool full = (j0 + BN <= p.l_k) && ((long long)j0 - wb >= p.dlo) &&
                          ((long long)(j0 + BN - 1) - wa <= p.dhi);
        if (!full && D == 128) {
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
              const int rel = j - qi;
              const bool ok = rel >= p.dlo && rel <= p.dhi && j < p.l_k;
              sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
            }
        } else if (!full) {
          // Score (kb, r) is key j0 + 4 half + c, c = 32 kb + 8 (r / 4) + r % 4.
          // This lane's allowed c form one interval lo64 .. hi64 (from
          // dlo <= j - qi <= dhi and j < l_k, clamped to the tile), turned
          // into a 64-bit mask once per tile; each score then costs one
          // sign-extending bit extract and one bit select, a third of the
          // VALU work of testing the bounds one by one, which matters where
          // masked tiles are common (the sliding window at d = 64).  At
          // d = 128 the per-bound form is kept: with it the compiler
          // schedules the whole step better (measured: the mask form costs
          // C2 and C5 ~10%).
          const long long base = (long long)qi - j0 - 4 * half;
          const long long lo64 = max(base + p.dlo, 0LL);
          const long long hi64 = min(min(base + p.dhi, (long long)p.l_k - 1 - j0 - 4 * half),
                                     (long long)BN - 1);
          const bool none = hi64 < lo64;
          // (no compare-to-VCC chain, which costs a wait state per score)
          const int lo_c = (int)min(lo64, 63LL);  // shift counts kept in range
          const int hi_c = (int)max(hi64, -1LL);
          const uint64_t upto = hi_c >= 63 ? ~0ULL : ((1ULL << (hi_c + 1)) - 1);
          const uint64_t mask = none ? 0ULL : upto & (~0ULL << lo_c);
          const uint32_t mw[2] = {(uint32_t)mask, (uint32_t)(mask >> 32)};
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 8 * (r >> 2) + (r & 3);  // bit within mw[kb]
              const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)mw[kb], c, 1);
              sacc[kb][r] = __uint_as_float((__float_as_uint(sacc[kb][r]) & keep) |
                                            (0xff800000u & ~keep));
            }
        }
        float mx = kNegInf;
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = pair_max(mx);
        const float mt = mx * p.c;  // c > 0: -inf stays -inf
        // keep the stale max unless this tile's max exceeds it by the slack;
        // lanes that keep it have alpha = 1 (their m may still be -inf)
        const bool grow = mt > m + kRescaleSlack;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
        m = grow ? mt : m;
        const float muse = (m == kNegInf) ? 0.f : m;
        u32x4_t pf[NPS];
        float rs = 0.f;
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.c, -muse));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], p.c, -muse));
            const uint32_t pk = pack_bf16x2(p0, p1);
            pf[2 * kb + (r >> 3)][(r & 7) >> 1] = pk;
            // row sum of the bf16 weights the P.V MFMA actually applies
            rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                                 __builtin_bit_cast(bf16x2_t, 0x3f803f80u),
                                                 rs, false);
          }
        lsum = lsum * alpha + rs;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
  #pragma unroll
          for (int db = 0; db < NDB; ++db)
  #pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        // ---- O^T += V^T P^T, V^T read transposed out of the row-major tile
  #pragma unroll
        for (int t = 0; t < NPS; ++t)
  #pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(vl + t * 16 * RB + (va ^ (64u * db))));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(vl + t * 16 * RB + 8 * RB + (va ^ (64u * db + kVC))));
            const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
            const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
            const u32x4_t a = {l2[0], l2[1], h2[0], h2[1]};
            oacc[db] = mfma32x32x16(a, pf[t], oacc[db]);
          }
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's DMA landed
      __syncthreads();
    };

    // this group's tiles: kt_begin + grp + KSPLIT u; every group runs the same
    // number of steps (and barriers), idling past its last tile
    const int kt_first = kt_begin + grp;
    const int n_steps = (kt_end - kt_begin + KSPLIT - 1) / KSPLIT;
    if (kt_begin < kt_end) {
      if (kt_first < kt_end) load_tile(kt_first, k_lds0[grp], v_lds0[grp]);
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
    // unrolled by two so that every buffer reference is a fixed LDS object
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

    float ltot = pair_sum(lsum);
    if constexpr (KSPLIT == 2) {
      // ---- merge group 1's partial rows into group 0's (both shift to the
      // larger max) through LDS in one round: group 1 stores its O
      // accumulators (float4 f = 4 db + r4 of lane wl at (f, wl), spread over
      // the two V buffers) and (m, l) (group 1's slot of the second K buffer)
      const int wl = wave * 64 + lane;
      float4* xo0 = reinterpret_cast<float4*>(&v_lds0[0][0]);
      float4* xo1 = reinterpret_cast<float4*>(&v_lds1[0][0]);
      float2* xml = reinterpret_cast<float2*>(&k_lds1[1][0]) + wl;
      static_assert(NDB * 2 * kThreads * 16 <= KSPLIT * BN * D * 2, "exchange fits");
      if (grp == 1) {
#pragma unroll
        for (int f = 0; f < 4 * NDB; ++f) {
          const float4 x = {oacc[f / 4][4 * (f % 4)], oacc[f / 4][4 * (f % 4) + 1],
                            oacc[f / 4][4 * (f % 4) + 2], oacc[f / 4][4 * (f % 4) + 3]};
          (f < 2 * NDB ? xo0 : xo1)[(f % (2 * NDB)) * kThreads + wl] = x;
        }
        *xml = make_float2(m, ltot);
      }
      __syncthreads();
      if (grp == 1) return;
      const float2 ml1 = *xml;
      const float mm = fmaxf(m, ml1.x);
      const float w0 = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - mm);
      const float w1 = (ml1.x == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml1.x - mm);
#pragma unroll
      for (int f = 0; f < 4 * NDB; ++f) {
        const float4 x = (f < 2 * NDB ? xo0 : xo1)[(f % (2 * NDB)) * kThreads + wl];
        oacc[f / 4][4 * (f % 4)] = oacc[f / 4][4 * (f % 4)] * w0 + x.x * w1;
        oacc[f / 4][4 * (f % 4) + 1] = oacc[f / 4][4 * (f % 4) + 1] * w0 + x.y * w1;
        oacc[f / 4][4 * (f % 4) + 2] = oacc[f / 4][4 * (f % 4) + 2] * w0 + x.z * w1;
        oacc[f / 4][4 * (f % 4) + 3] = oacc[f / 4][4 * (f % 4) + 3] * w0 + x.w * w1;
      }
      ltot = ltot * w0 + ml1.y * w1;
      m = mm;
    }

    if constexpr (ACC) {
      // ---- epilogue: merge (O / l, LSE) into the accumulator rows.  The
      // weights follow the log1p form of the chunk merge, with the same -inf
      // guards as attn_merge: a block row with no allowed key leaves the row
      // alone (or clears it to O = 0 when the accumulator row is at -inf
      // too), an accumulator row at -inf is replaced (never multiplied, so
      // whatever it holds cannot leak).  The block's rows pass through LDS
      // in fp32, 16 rows per round in this wave's own 8 KB slice of the
      // first K buffer slots, so that every accumulator access is a whole
      // 512-byte row.
      const float muse = (m == kNegInf) ? 0.f : m;
      const float lb = ltot > 0.f ? (muse + __log2f(ltot)) * kLn2 : kNegInf;
      const size_t li = (size_t)head * p.l_q + min(qi, last_row);
      const float la = p.lse_acc[li];
      int mode = la == kNegInf ? 3 : 0;  // 0 keep, 1 replace, 2 weighted sum, 3 clear
      float wa = 0.f, wb = 0.f;
      if (lb != kNegInf) {
        if (la == kNegInf) {
          mode = 1;
          wb = 1.f / ltot;
          if (half == 0 && qi <= last_row) p.lse_acc[li] = lb;
        } else {
          mode = 2;
          const float mx = fmaxf(la, lb), mn = fminf(la, lb);
          const float ln = mx + log1pf(expf(mn - mx));
          wa = expf(la - ln);
          wb = expf(lb - ln) / ltot;
          if (half == 0 && qi <= last_row) p.lse_acc[li] = ln;
        }
      }
      const uint32_t ecol = (uint32_t)lane & 31u, ehalf = (uint32_t)lane >> 5;
      float* stage = reinterpret_cast<float*>(
          (wave < 2 ? &k_lds0[0][0] : &k_lds1[0][0]) + (wave & 1) * 32 * RB);
      constexpr int CH = D / 4;  // 16-byte chunks of an fp32 row
      static_assert(16 * CH * 16 <= 32 * RB, "16 fp32 rows fit the wave's slice");
#pragma unroll
      for (int round = 0; round < 2; ++round) {
        if ((int)(ecol >> 4) == round) {
          const uint32_t row = ecol & 15u;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const uint32_t c = (uint32_t)(8 * db + 2 * r4) + ehalf;
              const f32x4_t x = {oacc[db][4 * r4] * wb, oacc[db][4 * r4 + 1] * wb,
                                 oacc[db][4 * r4 + 2] * wb, oacc[db][4 * r4 + 3] * wb};
              *reinterpret_cast<f32x4_t*>(stage + row * D + 4 * (c ^ (2u * row % CH))) = x;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int it = 0; it < 16 * CH / 64; ++it) {
          const int k = it * 64 + lane;
          const int rr = k / CH, c = k % CH;
          const int src = 16 * round + rr;  // the lane that holds this row
          const int rmode = __shfl(mode, src);
          const float rwa = __shfl(wa, src);
          const int i = iw + src;
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(
              stage + rr * D + 4 * (c ^ (2 * rr % CH)));
          if (i <= last_row && rmode != 0) {
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(
                p.acc + ((size_t)b * p.l_q + i) * q_row + (size_t)hq * D + 4 * c);
            *dst = rmode == 1 ? x : rmode == 3 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : *dst * rwa + x;
          }
        }
      }
    } else {
      // ---- epilogue: normalise, write O (bf16) and LSE (natural log).  The
      // wave's 32 O rows pass through LDS (its own 32-row slice of the first
      // slot of the K buffers, chunks XOR-swizzled by row as the tiles are) so
      // that every global store writes whole rows.
      {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        const uint32_t ln = (uint32_t)lane;
        const uint32_t ecol = ln & 31u, ehalf = ln >> 5;
        unsigned char* stage = (wave < 2 ? &k_lds0[0][0] : &k_lds1[0][0]) + (wave & 1) * 32 * RB;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            u32x2_t w;
            w[0] = pack_bf16x2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv);
            w[1] = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
            const uint32_t c = (uint32_t)(4 * db + r4) ^ chunk_swz<D>(ecol);
            *reinterpret_cast<u32x2_t*>(stage + ecol * RB + c * 16 + 8 * ehalf) = w;
          }
        // the wave reads back what its own lanes wrote: LDS operations of one
        // wave complete in order once counted down
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
        for (int x = 0; x < 32 / RPI; ++x) {
          const int r = x * RPI + (int)(ln / CPR);
          const uint32_t c = (ln % CPR) ^ chunk_swz<D>((uint32_t)r);
          const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stage + r * RB + c * 16);
          if (iw + r <= last_row)
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(
                p.o + ((size_t)b * p.l_q + iw + r) * q_row + (size_t)hq * D + 8 * (ln % CPR)));
        }
        if (half == 0 && qi <= last_row) {
          const float muse = (m == kNegInf) ? 0.f : m;
          p.lse[(size_t)head * p.l_q + qi] =
              ltot > 0.f ? (muse + __log2f(ltot)) * kLn2 : kNegInf;
        }
      }
    }
  };

  int unit, head;
  map_block(p, unit, head);
  // pairing: the shorter tile r first, then n_qtiles-1-r (once if the same).
  // Under a causal mask both read keys from 0 on, so the longer tile finds
  // the shorter one's keys still in L2 (the other order fetched ~16 MB more
  // per launch on the 2 x 2048-token, 16-head workload).
  const int n_tiles = p.pairs ? (unit == p.n_qtiles - 1 - unit ? 1 : 2) : 1;
  for (int ti = 0; ti < n_tiles; ++ti) {
    const int tile = p.pairs ? (ti == 1 ? p.n_qtiles - 1 - unit : unit) : unit;
    // the previous tile's merge and output staging read LDS buffers that
    // this tile's first loads overwrite
    if (ti > 0) __syncthreads();
    fwd_tile(tile, head);
  }
}

// ---------------------------------------------------------------- fp32 path
//
// fp32 inputs: a SIMT kernel (fp32 FMA), 64 query rows per workgroup, four
// lanes per row each owning D/4 dims (float4 chunks c, c+4, c+8, ...).  Keys
// are staged 64 at a time in LDS and consumed in groups of 16 with the same
// online-softmax update as the bf16 kernel.
struct FwdF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int l_q, l_k, h, h_kv, grp;
  int n_heads;
  float c;          // |scale| * log2(e)
  int neg_scale;    // 1: scale < 0 (Q enters negated)
  int dlo, dhi;
  float* acc;       // ACC: the fp32 ring accumulator merged into
  float* lse_acc;
};

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 64;

template <int D, bool ACC>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdF32Params p) {
  constexpr int NC = D / 16;  // float4 chunks per lane
  __shared__ f32x4_t ks[kF32Keys * (D / 4)];
  __shared__ f32x4_t vs[kF32Keys * (D / 4)];

  const int tid = threadIdx.x;
  const int c = tid & 3;
  const int row = tid >> 2;
  const int tile = blockIdx.x / p.n_heads;
  const int head = blockIdx.x - tile * p.n_heads;
  const int b = head / p.h;
  const int hq = head - b * p.h;
  const int g = hq / p.grp;
  const int last_row = p.l_q - 1;
  const int i0 = tile * kF32Rows;
  const int qi = i0 + row;

  const long long jlo = max(0LL, (long long)i0 + p.dlo);
  const long long jhi = min((long long)p.l_k - 1,
                            (long long)min(i0 + kF32Rows - 1, last_row) + p.dhi);

  const size_t q_row = (size_t)p.h * D;
  const f32x4_t* qptr = reinterpret_cast<const f32x4_t*>(
      p.q + ((size_t)b * p.l_q + min(qi, last_row)) * q_row + (size_t)hq * D);
  f32x4_t qv[NC];
  f32x4_t ov[NC];
#pragma unroll
  for (int m4 = 0; m4 < NC; ++m4) {
    qv[m4] = p.neg_scale ? -qptr[c + 4 * m4] : qptr[c + 4 * m4];  // fold the sign
    ov[m4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float m = kNegInf, lsum = 0.f;

  const size_t kv_row = (size_t)p.h_kv * D;
  const float* kbase = p.k + (size_t)b * p.l_k * kv_row + (size_t)g * D;
  const float* vbase = p.v + (size_t)b * p.l_k * kv_row + (size_t)g * D;

  if (jlo <= jhi) {
    for (long long j0 = (jlo / kF32Keys) * kF32Keys; j0 <= jhi; j0 += kF32Keys) {
      __syncthreads();
      for (int e = tid; e < kF32Keys * (D / 4); e += 256) {
        const int kr = e / (D / 4);
        const int c4 = e - kr * (D / 4);
        const long long j = min(j0 + kr, (long long)p.l_k - 1);
        ks[e] = reinterpret_cast<const f32x4_t*>(kbase + (size_t)j * kv_row)[c4];
        vs[e] = reinterpret_cast<const f32x4_t*>(vbase + (size_t)j * kv_row)[c4];
      }
      __syncthreads();
      for (int jg = 0; jg < kF32Keys; jg += 16) {
        float s[16];
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          float acc = 0.f;
#pragma unroll
          for (int m4 = 0; m4 < NC; ++m4) {
            const f32x4_t kk = ks[(jg + jj) * (D / 4) + c + 4 * m4];
            acc = fmaf(qv[m4][0], kk[0], acc);
            acc = fmaf(qv[m4][1], kk[1], acc);
            acc = fmaf(qv[m4][2], kk[2], acc);
            acc = fmaf(qv[m4][3], kk[3], acc);
          }
          acc += __shfl_xor(acc, 1);
          acc += __shfl_xor(acc, 2);
          const long long j = j0 + jg + jj;
          const long long rel = j - qi;
          const bool ok = j < p.l_k && rel >= p.dlo && rel <= p.dhi;
          s[jj] = ok ? acc : kNegInf;
          mx = fmaxf(mx, s[jj]);
        }
        const float mt = (mx == kNegInf) ? kNegInf : mx * p.c;
        const float mnew = fmaxf(m, mt);
        const float muse = (mnew == kNegInf) ? 0.f : mnew;
        const float alpha = exp2f(m - muse);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int m4 = 0; m4 < NC; ++m4) ov[m4] *= alpha;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float pj = (s[jj] == kNegInf) ? 0.f : exp2f(fmaf(s[jj], p.c, -muse));
          lsum += pj;
#pragma unroll
          for (int m4 = 0; m4 < NC; ++m4) {
            const f32x4_t vv = vs[(jg + jj) * (D / 4) + c + 4 * m4];
            ov[m4][0] = fmaf(pj, vv[0], ov[m4][0]);
            ov[m4][1] = fmaf(pj, vv[1], ov[m4][1]);
            ov[m4][2] = fmaf(pj, vv[2], ov[m4][2]);
            ov[m4][3] = fmaf(pj, vv[3], ov[m4][3]);
          }
        }
      }
    }
  }
  if (qi <= last_row) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float muse = (m == kNegInf) ? 0.f : m;
    const float lse_blk = lsum > 0.f ? (muse + log2f(lsum)) * kLn2 : kNegInf;
    const size_t orow = ((size_t)b * p.l_q + qi) * q_row + (size_t)hq * D;
    const size_t li = (size_t)head * p.l_q + qi;
    if (!ACC) {
      f32x4_t* optr = reinterpret_cast<f32x4_t*>(p.o + orow);
#pragma unroll
      for (int m4 = 0; m4 < NC; ++m4) optr[c + 4 * m4] = ov[m4] * inv;
      if (c == 0) p.lse[li] = lse_blk;
    } else {
      // the merge of (O / l, lse_blk) into the accumulator row, with the
      // merge kernel's weights and -inf guards: an empty block keeps the
      // row (or clears it when the row is empty too), an empty accumulator
      // row takes the block
      f32x4_t* aptr = reinterpret_cast<f32x4_t*>(p.acc + orow);
      const float a = p.lse_acc[li];  // read by all four lanes before lane 0 writes
      if (lse_blk == kNegInf) {
        if (a == kNegInf) {
#pragma unroll
          for (int m4 = 0; m4 < NC; ++m4) aptr[c + 4 * m4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      } else if (a == kNegInf) {
#pragma unroll
        for (int m4 = 0; m4 < NC; ++m4) aptr[c + 4 * m4] = ov[m4] * inv;
        if (c == 0) p.lse_acc[li] = lse_blk;
      } else {
        const float mx = fmaxf(a, lse_blk);
        const float mn = fminf(a, lse_blk);
        const float lse = mx + log1pf(expf(mn - mx));
        const float wa = expf(a - lse);
        const float wb = expf(lse_blk - lse) * inv;
#pragma unroll
        for (int m4 = 0; m4 < NC; ++m4) aptr[c + 4 * m4] = aptr[c + 4 * m4] * wa + ov[m4] * wb;
        if (c == 0) p.lse_acc[li] = lse;
      }
    }
  }
}

// Workgroup schedule of the bf16 kernel:
//  * kOneGroup: one q tile per 4-wave workgroup, two workgroups per CU;
//  * kSplit: one q tile per 8-wave workgroup whose two key groups share the
//    tile's keys, one workgroup per CU (half the time per tile);
//  * kPairs: as kSplit, each workgroup taking q tiles n_qtiles-1-r and r.
// The choice minimises an estimate of the makespan in units of one tile's
// time on one 4-wave slot: max(longest workgroup, total work / slots).  The
// 8-wave workgroup is charged 8% more per tile (its eight waves meet at every
// barrier, so the MFMA and VALU phases of the two waves on a SIMD overlap
// less than those of two independent workgroups).
enum class FwdSchedule { kOneGroup, kSplit, kPairs };

constexpr int kCUs = 256;

int key_tiles(const FwdParams& p, int tile) {
  const long long i0 = (long long)tile * kBM;
  const long long jlo = std::max(0LL, i0 + p.dlo);
  const long long jhi = std::min((long long)p.l_k - 1,
                                 std::min(i0 + kBM - 1, (long long)p.l_q - 1) + p.dhi);
  return jlo <= jhi ? (int)(jhi / 64 - jlo / 64 + 1) : 0;
}

FwdSchedule pick_schedule(const FwdParams& p) {
  const int nt = p.n_qtiles;
  long long max1 = 0, sum1 = 0, max2 = 0, sum2 = 0, maxp = 0, sump = 0;
  for (int t = 0; t < nt; ++t) {
    const long long len = key_tiles(p, t);
    max1 = std::max(max1, len);
    sum1 += len;
    max2 = std::max(max2, (len + 1) / 2);
    sum2 += (len + 1) / 2;
  }
  for (int r = 0; r < (nt + 1) / 2; ++r) {
    const int a = nt - 1 - r;
    const long long len = (key_tiles(p, a) + 1) / 2 + (a != r ? (key_tiles(p, r) + 1) / 2 : 0);
    maxp = std::max(maxp, len);
    sump += len;
  }
  const double heads = p.n_heads;
  const double e1 = std::max((double)max1, sum1 * heads / (2.0 * kCUs));
  const double e2 = 1.08 * std::max((double)max2, sum2 * heads / kCUs);
  const double ep = 1.08 * std::max((double)maxp, sump * heads / kCUs);
  if (ep < e1 && ep <= e2) return FwdSchedule::kPairs;
  return e2 < e1 ? FwdSchedule::kSplit : FwdSchedule::kOneGroup;
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v,
                           void* out, float* lse, const AttnShape& s,
                           hipStream_t stream, float* acc, float* lse_acc) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.acc = acc;
  p.lse_acc = lse_acc;
  p.l_q = s.l_q;
  p.l_k = s.l_k;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  p.n_heads = s.n * s.h;
  p.n_qtiles = (s.l_q + kBM - 1) / kBM;
  p.xcd_groups = ((s.n * s.h_kv) % 8 == 0) ? 1 : 0;
  p.reverse = s.causal ? 1 : 0;
  p.c = (s.scale == 0.f ? 1.f : fabsf(s.scale)) * kLog2e;
  p.q_and = s.scale == 0.f ? 0u : 0xffffffffu;
  p.q_xor = s.scale < 0.f ? 0x80008000u : 0u;
  p.dlo = s.dlo;
  p.dhi = s.dhi;
  const FwdSchedule sch = pick_schedule(p);
  p.pairs = sch == FwdSchedule::kPairs ? 1 : 0;
  p.n_units = p.pairs ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  dim3 grid((unsigned)p.n_units * (unsigned)p.n_heads);
  const bool split = sch != FwdSchedule::kOneGroup;
  const dim3 block(split ? 2 * kThreads : kThreads);
  if (acc == nullptr) {
    if (split) {
      if (s.d == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, 2, false>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 2, false>), grid, block, 0, stream, p);
    } else {
      if (s.d == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, 1, false>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 1, false>), grid, block, 0, stream, p);
    }
  } else {
    if (split) {
      if (s.d == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, 2, true>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 2, true>), grid, block, 0, stream, p);
    } else {
      if (s.d == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, 1, true>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 1, true>), grid, block, 0, stream, p);
    }
  }
  return hipGetLastError();
}

const char* fwd_bf16_kernel_name(const AttnShape& s, bool acc) {
  FwdParams p;
  p.l_q = s.l_q;
  p.l_k = s.l_k;
  p.n_heads = s.n * s.h;
  p.n_qtiles = (s.l_q + kBM - 1) / kBM;
  p.dlo = s.dlo;
  p.dhi = s.dhi;
  const int split = pick_schedule(p) != FwdSchedule::kOneGroup ? 1 : 0;
  static const char* const names[2][2][2] = {
      {{"fwd_bf16_kernel<64, 64, 1, false>", "fwd_bf16_kernel<64, 64, 1, true>"},
       {"fwd_bf16_kernel<64, 64, 2, false>", "fwd_bf16_kernel<64, 64, 2, true>"}},
      {{"fwd_bf16_kernel<128, 64, 1, false>", "fwd_bf16_kernel<128, 64, 1, true>"},
       {"fwd_bf16_kernel<128, 64, 2, false>", "fwd_bf16_kernel<128, 64, 2, true>"}}};
  return names[s.d == 128 ? 1 : 0][split][acc ? 1 : 0];
}

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v,
                          void* out, float* lse, const AttnShape& s,
                          hipStream_t stream, float* acc, float* lse_acc) {
  FwdF32Params p;
  p.q = static_cast<const float*>(q);
  p.k = static_cast<const float*>(k);
  p.v = static_cast<const float*>(v);
  p.o = static_cast<float*>(out);
  p.lse = lse;
  p.l_q = s.l_q;
  p.l_k = s.l_k;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  p.n_heads = s.n * s.h;
  p.c = fabsf(s.scale) * kLog2e;
  p.neg_scale = s.scale < 0.f ? 1 : 0;
  p.dlo = s.dlo;
  p.dhi = s.dhi;
  p.acc = acc;
  p.lse_acc = lse_acc;
  const unsigned tiles = (unsigned)((s.l_q + kF32Rows - 1) / kF32Rows);
  dim3 grid(tiles * (unsigned)p.n_heads);
  dim3 block(256);
  if (acc) {
    if (s.d == 128)
      hipLaunchKernelGGL((fwd_f32_kernel<128, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_f32_kernel<64, true>), grid, block, 0, stream, p);
  } else if (s.d == 128) {
    hipLaunchKernelGGL((fwd_f32_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((fwd_f32_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace bea
