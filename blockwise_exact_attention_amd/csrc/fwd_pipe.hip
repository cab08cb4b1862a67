// Exact attention forward for gfx950 with a software pipeline inside every
// wave: bf16 MFMA with fp32 accumulation, online softmax, 32 query rows per
// wave, two waves per SIMD.
//
// What is computed follows the pages "picotron/parallel/context_parallel.py"
// (ring_attention_forward: S = scale * Q K^T, causal mask, LSE = log sum exp,
// O = softmax(S) V; RingAttention._repeat_kv for grouped heads) and
// "flash_sharding.py" (ring_fwd: the (O, LSE) pair per query row, a row with
// no allowed key gives O = 0 and LSE = -inf; the log1p merge, which the
// online softmax applies per key tile; and the loop over key/value chunks
// with their absolute offsets, which the multi-chunk form runs in one
// launch).
//
// Layout (one workgroup of 8 waves per CU; 132 KB of LDS at KSPLIT = 2,
// 64 KB at KSPLIT = 1):
//  * A wave owns 32 query rows of one head.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows from LDS are the A
//    operand, the wave's Q rows stay in VGPRs as the B operand.  In the
//    result a lane holds one query (lane % 32) and 32 of the tile's 64 keys,
//    so a row max needs one exchange between the two half-waves.
//  * O^T += V^T P^T takes the bf16 P straight out of the S^T registers as
//    its B operand (the contraction order over keys is free); V^T is read
//    out of the row-major V tile with transposing LDS reads.
//  * KSPLIT = 2: two key groups of four waves cover the same 128 rows and
//    take alternate key tiles, each with its own LDS buffers; their partial
//    rows are merged through LDS at the end, each group finishing half of
//    the head dims.  KSPLIT = 1: one group of eight waves covers 256 rows.
//  * Per key tile a wave runs two phases, each a fixed sequence of slots
//    pinned in place (an empty asm on every softmax result, a scheduling
//    barrier between slots):
//      phase 1: the 16 (d = 128) MFMAs of S_{u+1} = K_{u+1} Q^T, with the
//               exponentials, bf16 packing and row sums of tile u between
//               them, and this wave's share of the next tiles' loads;
//      phase 2: the 16 MFMAs of O += P_u V_u, with the row max and exponent
//               arguments of tile u+1 between them.
//    The softmax of one tile so runs in the shadow of the products of its
//    neighbours instead of between them.  Boundary tiles (causal diagonal,
//    window edges, ragged ends) get a mask pass before phase 2.
//  * K and V tiles of 64 keys are double-buffered in LDS and filled by
//    direct buffer-to-LDS loads; K runs one tile ahead of V.  One barrier
//    per tile.  KSPLIT = 2: the workgroup stages the q tile's rows in LDS
//    once (both key groups need them) and every wave reads its fragment
//    from there; KSPLIT = 1: each wave loads its own rows straight into
//    registers.
//  * The running max is updated lazily (rescale only when a tile's max
//    exceeds it by a slack), so O is rarely touched outside the products.
//  * Normalised O leaves through LDS as row-contiguous stores.  The ACC
//    instantiations merge (O, LSE) into a float32 accumulator instead.
//  * MULTI: the key tiles are those of up to kMaxChunks key/value chunks,
//    each with its own pointers, length and mask bounds, visited in order by
//    one online softmax.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace bea {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;             // keys per tile
constexpr float kSlack = 8.f;       // lazy rescale threshold (log2 units)

struct PipeParams {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  float* acc;      // ACC: fp32 accumulator O [n, l_q, h, d]
  float* lse_acc;  // ACC: its LSE [n, h, l_q] (natural log)
  FwdChunk ch[kMaxChunks];
  int n_chunks;
  int l_q, h, h_kv, grp;
  int n_heads;     // n * h
  int n_qtiles;
  int n_units;     // workgroups per head: n_qtiles, or ceil(n_qtiles / 2) paired
  int pairs;       // 1: workgroup r takes q tiles r and n_qtiles-1-r
  int xcd_groups;  // 1: keep the workgroups of one key/value head on one XCD
  int reverse;     // 1: the last (longest, under causal) q tiles first
  float c;         // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t q_and;  // Q fragment mask: 0 when scale == 0
  uint32_t q_xor;  // Q sign flip: 0x80008000 when scale < 0
};

// blockIdx.x -> (work unit, flattened head b*h + hq).  Workgroups go to the
// 8 XCDs round-robin by id and each XCD has its own L2: when the key/value
// groups split evenly over the XCDs, every workgroup that reads one
// key/value head gets an id of the same residue mod 8.  Under causal
// masking the last q tiles see the most keys; they get the lowest ids.
__device__ __forceinline__ void map_block(const PipeParams& p, int& unit, int& head) {
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

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// keep a value where it is computed (no sinking past the slot it is placed in)
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Key tiles of one q tile in one chunk: [beg, beg + cnt).
struct TileSpan {
  int beg, cnt;
};

__device__ __forceinline__ TileSpan chunk_span(const FwdChunk& ch, int i_first, int i_last) {
  const long long jlo = max(0LL, (long long)i_first + ch.dlo);
  const long long jhi = min((long long)ch.l_k - 1, (long long)i_last + ch.dhi);
  if (jlo > jhi) return TileSpan{0, 0};
  const int b = (int)(jlo / kBN);
  return TileSpan{b, (int)(jhi / kBN) - b + 1};
}

// Where virtual tile v (counted over the chunks in order) lives.
struct TileRef {
  int c;    // chunk
  int kt;   // tile index within the chunk
};

template <bool MULTI>
__device__ __forceinline__ TileRef locate(const PipeParams& p, int v, int i_first, int i_last) {
  if (!MULTI) return TileRef{0, chunk_span(p.ch[0], i_first, i_last).beg + v};
  int c = 0;
  for (; c < p.n_chunks - 1; ++c) {
    const TileSpan s = chunk_span(p.ch[c], i_first, i_last);
    if (v < s.cnt) return TileRef{c, s.beg + v};
    v -= s.cnt;
  }
  return TileRef{c, chunk_span(p.ch[c], i_first, i_last).beg + v};
}

template <int D, int KSPLIT, bool ACC, bool MULTI>
__global__ __launch_bounds__(kThreads, 1) void fwd_pipe_kernel(PipeParams p) {
  constexpr int WPG = kWaves / KSPLIT;          // waves per key group
  constexpr int QROWS = 32 * WPG;               // query rows per q tile
  constexpr int RB = D * 2;                     // bytes per tile row
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int TILE = kBN * RB;
  constexpr int RPD = 1024 / RB;                // rows one wave-wide load writes
  constexpr int KV_DMA = kBN / RPD / WPG;       // loads per wave per K (or V) tile
  constexpr int NKB = 2;         // 32-key blocks per tile
  constexpr int NDS = D / 16;    // S^T MFMA k steps
  constexpr int NDB = D / 32;    // 32-dim blocks of O^T
  constexpr int NPS = 4;         // 16-key slices (O^T MFMA k steps)
  constexpr int NSLOT = NKB * NDS;   // phase-1 slots, one product each
  constexpr int NSLOT2 = NPS * NDB;  // phase-2 slots, one product each
  constexpr uint32_t kVC = D == 128 ? 32u : 16u;
  static_assert(KV_DMA >= 1, "loads");
  // the swizzle repeats every 16 rows: with rows stepping by a multiple of
  // 16 between a wave's loads, one lane offset serves them all
  static_assert((WPG * RPD) % 16 == 0 && (kWaves * RPD) % 16 == 0, "swizzle period");

  // the key groups' (m, l) exchange at the end of a q tile
  __shared__ float2 xml_lds[KSPLIT == 2 ? kWaves * 64 : 1];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[KSPLIT][TILE];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds1[KSPLIT][TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[KSPLIT][TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds1[KSPLIT][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / WPG;   // key group
  const int wr = wave_all % WPG;    // 32-row block of the q tile
  const int half = lane >> 5;
  const int col = lane & 31;

  uint32_t ka0, va0;
  lds_read_bases<D>(lane, ka0, va0);
  // per-lane LDS byte offsets of the operand reads within a K or V buffer
  // array, the key group's slot included: a read is one of these registers
  // plus the buffer's address and an immediate
  uint32_t kad[NDS], vad[NDB][2];
#pragma unroll
  for (int s = 0; s < NDS; ++s) kad[s] = (uint32_t)grp * TILE + (ka0 ^ (32u * s));
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    vad[db][0] = (uint32_t)grp * TILE + (va0 ^ (64u * db));
    vad[db][1] = (uint32_t)grp * TILE + 8 * RB + (va0 ^ (64u * db + kVC));
  }

  int unit, head;
  map_block(p, unit, head);
  const int b = head / p.h;
  const int hq = head - b * p.h;
  const int g = hq / p.grp;
  const size_t q_row = (size_t)p.h * D;
  const uint32_t q_row_b = (uint32_t)q_row * 2u;
  const size_t kv_row = (size_t)p.h_kv * D;
  const uint32_t kv_row_b = (uint32_t)kv_row * 2u;
  const int last_row = p.l_q - 1;

  // lane offsets of the loads: load x of wave w writes rows
  // (x W + w) RPD + lane / CPR of its tile; the lane fetches the logical
  // chunk the swizzle puts at its slot
  const uint32_t lrow = (uint32_t)(lane / CPR);
  const uint32_t lchunk = (uint32_t)(lane % CPR);
  const uint32_t kv_voff =
      lrow * kv_row_b + ((lchunk ^ chunk_swz<D>((uint32_t)wr * RPD + lrow)) * 16u);

  // one q tile: prologue, key loop, merge of the key groups, epilogue
  auto fwd_tile = [&](const int tile) {
    const int i0 = tile * QROWS;
    const int i_last = min(i0 + QROWS, p.l_q) - 1;
    const int iw = i0 + wr * 32;  // this wave's first row
    const int qi = iw + col;      // this lane's query row

    // key tiles of this q tile over all chunks; group grp takes the virtual
    // tiles grp, grp + KSPLIT, ...
    int total = 0;
    if (MULTI) {
      for (int c = 0; c < p.n_chunks; ++c) total += chunk_span(p.ch[c], i0, i_last).cnt;
    } else {
      total = chunk_span(p.ch[0], i0, i_last).cnt;
    }
    const int n_g = (total - grp + KSPLIT - 1) / KSPLIT;   // this group's tiles
    const int n_steps = (total + KSPLIT - 1) / KSPLIT;     // group 0's (the most)

    // ---- cursor over the virtual tiles: chunk c, tile kt within it, and
    // the end of the chunk's span for this q tile.  Valid while kt < end (a
    // cursor only stops short of its chunk's end in the last chunk).  The
    // key loop moves each cursor KSPLIT tiles per step, crossing into the
    // next chunks with non-empty spans: constant scalar work per step.
    struct Cur {
      int c, kt, end;
    };
    auto cur_at = [&](int v) {
      const TileRef t = locate<MULTI>(p, v, i0, i_last);
      const TileSpan sp = chunk_span(p.ch[t.c], i0, i_last);
      return Cur{t.c, t.kt, sp.beg + sp.cnt};
    };
    auto cur_next = [&](Cur x) {
      x.kt += KSPLIT;
      if (MULTI) {
        while (x.kt >= x.end && x.c + 1 < p.n_chunks) {
          const int over = x.kt - x.end;
          ++x.c;
          const TileSpan sp = chunk_span(p.ch[x.c], i0, i_last);
          x.kt = sp.beg + over;
          x.end = sp.beg + sp.cnt;
        }
      }
      return x;
    };

    // ---- buffer resource of one K or V tile; past the last tile a
    // zero-length range, whose loads write zeros into a buffer nobody reads
    auto kv_rsrc = [&](const Cur& x, bool is_v) {
      int bytes = 0;
      const uint16_t* base = p.ch[0].k;
      if (x.kt < x.end) {
        const FwdChunk& ch = p.ch[x.c];
        const long long rows = (long long)ch.l_k - (long long)x.kt * kBN;
        bytes = (int)min(rows * (long long)kv_row_b, 0x7fffffffLL);
        base = (is_v ? ch.v : ch.k) + ((size_t)b * ch.l_k + (size_t)x.kt * kBN) * kv_row +
               (size_t)g * D;
      }
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes,
                                               0x00020000);
    };
    // load x of this wave's share of a tile
    auto dma_kv = [&](__amdgpu_buffer_rsrc_t rs, unsigned char* dst, int x) {
      const uint32_t row0 = (uint32_t)((x * WPG + wr) * RPD);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + row0 * RB), 16, kv_voff,
                                               row0 * kv_row_b, 0, 0);
    };

    // ---- prologue: the wave's Q fragment (rows past the end read as
    // zeros), K and V of the first tile, K of the second.  Lane (col, half)
    // holds row iw + col, dims 16 s + 8 half .. + 7 in qf[s]: the B operand
    // of the score products, resident for the whole key loop.  With one key
    // group it comes straight into registers (each wave reads only its own
    // rows).
    u32x4_t qf[NDS];
    {
      const long long rows = (long long)p.l_q - i0;
      const int bytes = (int)min(rows * (long long)q_row_b, 0x7fffffffLL);
      const uint16_t* base = p.q + ((size_t)b * p.l_q + i0) * q_row + (size_t)hq * D;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0,
                                                        bytes, 0x00020000);
      if constexpr (KSPLIT == 2) {
        // both key groups need the same 128 rows: the workgroup loads them
        // once, whole rows per load, into the second V buffers (first
        // written by the key loop's first step) in the tiles' swizzled
        // layout; every wave reads its fragment back after the barrier
        constexpr int QLOADS = QROWS / RPD / kWaves;
        static_assert(QLOADS >= 1 && QROWS * RB == KSPLIT * TILE, "Q staging");
        const uint32_t q_voff =
            lrow * q_row_b + ((lchunk ^ chunk_swz<D>((uint32_t)wave_all * RPD + lrow)) * 16u);
#pragma unroll
        for (int x = 0; x < QLOADS; ++x) {
          const uint32_t row0 = (uint32_t)((x * kWaves + wave_all) * RPD);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(&v_lds1[0][0] + row0 * RB),
                                                   16, q_voff, row0 * q_row_b, 0, 0);
        }
      } else {
        const uint32_t off = (uint32_t)(wr * 32 + col) * q_row_b + (uint32_t)half * 16u;
#pragma unroll
        for (int s = 0; s < NDS; ++s)
          qf[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 32u * s), 0, 0);
      }
    }
    // cursors of this group's first tile, of the tile whose V (and mask) the
    // first step needs, and of the tile whose K it loads
    const Cur cur0 = cur_at(grp);
    Cur curV = cur_next(cur0);
    Cur curK = cur_next(curV);
    // only Q and the first K tile before the first scores: V of the first
    // tile and K of the second are loaded between those products, so that
    // their latency hides behind the first tile's compute
    if (n_g > 0) {
      const auto rk = kv_rsrc(cur0, false);
#pragma unroll
      for (int x = 0; x < KV_DMA; ++x) dma_kv(rk, k_lds0[grp], x);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    if constexpr (KSPLIT == 2) {
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        qf[s] = *reinterpret_cast<const u32x4_t*>(&v_lds1[0][0] + (uint32_t)wr * 32u * RB +
                                                  (ka0 ^ (32u * s)));
    }

    // The sign of the scale is folded into Q (sign-bit flip, exact) and a
    // zero scale becomes Q = 0 with c = log2(e) (every allowed score is then
    // 0, as scale * q.k is), so c > 0 below and a masked score of -inf
    // always gives exp2(-inf) = 0.
#pragma unroll
    for (int s = 0; s < NDS; ++s) qf[s] = (qf[s] & p.q_and) ^ p.q_xor;

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = kNegInf;   // running max (log2 units)
    float lsum = 0.f;    // this lane's half of the row sum
    float alpha = 1.f;   // rescale factor of the latest max update
    f32x16_t sA[NKB], sB[NKB];  // scores / exponent arguments of two tiles
    u32x4_t pf[NPS];            // bf16 P of the tile in phase 2

    // mask of a tile for this wave: whether it is full (no mask work; wave
    // uniform, scalar arithmetic), else the lane's allowed key bits
    struct TileInfo {
      bool full;
      int j0, l_k, dlo, dhi;
    };
    auto tile_info = [&](const Cur& x) {
      const FwdChunk& ch = p.ch[x.c];
      TileInfo ti;
      ti.j0 = x.kt * kBN;
      ti.l_k = ch.l_k;
      ti.dlo = ch.dlo;
      ti.dhi = ch.dhi;
      ti.full = (ti.j0 + kBN <= ch.l_k) && ((long long)ti.j0 - (iw + 31) >= ch.dlo) &&
                ((long long)(ti.j0 + kBN - 1) - iw <= ch.dhi);
      return ti;
    };
    struct Mask {
      uint32_t w[NKB];
    };
    auto tile_bits = [&](const TileInfo& ti) {
      // score (kb, r) is key j0 + 4 half + c', c' = 32 kb + 8 (r / 4) + r % 4;
      // the allowed c' of this lane's row form one interval
      Mask mk;
      const long long base = (long long)qi - ti.j0 - 4 * half;
      const long long lo64 = max(base + ti.dlo, 0LL);
      const long long hi64 = min(min(base + ti.dhi, (long long)ti.l_k - 1 - ti.j0 - 4 * half),
                                 (long long)kBN - 1);
      const bool none = hi64 < lo64;
      const int lo_c = (int)min(lo64, 63LL);  // shift counts kept in range
      const int hi_c = (int)max(hi64, -1LL);
      const uint64_t upto = hi_c >= 63 ? ~0ULL : ((1ULL << (hi_c + 1)) - 1);
      const uint64_t bits = none ? 0ULL : upto & (~0ULL << lo_c);
      mk.w[0] = (uint32_t)bits;
      mk.w[1] = (uint32_t)(bits >> 32);
      return mk;
    };
    // boundary tile: masked scores become -inf (a sign-extending bit extract
    // and a bit select per score)
    auto apply_mask = [&](f32x16_t (&S)[NKB], const Mask& mk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cbit = 8 * (r >> 2) + (r & 3);
          const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)mk.w[kb], cbit, 1);
          S[kb][r] = __uint_as_float((__float_as_uint(S[kb][r]) & keep) | (0xff800000u & ~keep));
        }
    };

    // ---- softmax, first half (phase-2 work): row max, lazy rescale
    // decision, exponent arguments t = s c - m in place.  A wave issues in
    // order, so a VALU operation placed right after the one it depends on
    // stalls the products behind it: the work is cut into 13 stages, each
    // depending only on earlier stages, one stage per phase-2 slot.
    constexpr int NSTAGE_A = 13;
    struct SoftA {
      float l1[NKB][5];   // max3 of 15 of a key block's 16 scores
      float l2[NKB][2];
      float c, d, mt, diff, mnew, e;
      bool grow;
      float muse;
    };
    auto soft_a = [&](f32x16_t (&S)[NKB], int st, SoftA& z) {
      if (st < 2) {
        const int kb = st;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          z.l1[kb][i] = fmaxf(fmaxf(S[kb][3 * i], S[kb][3 * i + 1]), S[kb][3 * i + 2]);
          pin(z.l1[kb][i]);
        }
      } else if (st == 2) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          z.l2[kb][0] = fmaxf(fmaxf(z.l1[kb][0], z.l1[kb][1]), z.l1[kb][2]);
          z.l2[kb][1] = fmaxf(fmaxf(z.l1[kb][3], z.l1[kb][4]), S[kb][15]);
          pin(z.l2[kb][0]);
          pin(z.l2[kb][1]);
        }
      } else if (st == 3) {
        z.c = fmaxf(fmaxf(z.l2[0][0], z.l2[0][1]), z.l2[1][0]);
        pin(z.c);
      } else if (st == 4) {
        z.d = fmaxf(z.c, z.l2[1][1]);
        pin(z.d);
      } else if (st == 5) {
        z.d = pair_max(z.d);   // the row's max over the tile's 64 keys
        pin(z.d);
      } else if (st == 6) {
        // keep the stale max unless this tile's max exceeds it by the slack;
        // lanes that keep it have alpha = 1 (their m may still be -inf).
        // c > 0: -inf stays -inf.
        z.mt = z.d * p.c;
        z.grow = z.mt > m + kSlack;
        z.diff = m - z.mt;
        pin(z.mt);
        pin(z.diff);
      } else if (st == 7) {
        z.e = __builtin_amdgcn_exp2f(z.diff);
        z.mnew = z.grow ? z.mt : m;
        pin(z.e);
        pin(z.mnew);
      } else if (st == 8) {
        alpha = z.grow ? z.e : 1.f;
        m = z.mnew;
        z.muse = (m == kNegInf) ? 0.f : m;
        pin(alpha);
        pin(z.muse);
      } else {
        if (st == 9) lsum *= alpha;
        const int piece = st - 9;   // 8 of the 32 values
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = piece * 8 + e;
          float t = fmaf(S[idx >> 4][idx & 15], p.c, -z.muse);
          pin(t);
          S[idx >> 4][idx & 15] = t;
        }
      }
    };
    // ---- softmax, second half (phase-1 work): exponentials, bf16 P, row
    // sums.  Three stages per pair of values, one slot apart: the
    // exponentials of pair x, the packing of pair x - 1, the row sum of
    // pair x - 2 (PPS pairs per slot).
    constexpr int PPS = 16 / NSLOT;
    struct SoftB {
      float e[16][2];
      uint32_t pk[16];
      float rs;
    };
    auto soft_b_exp = [&](f32x16_t (&T)[NKB], int pr, SoftB& z) {
      const int kb = pr >> 3, r = 2 * (pr & 7);
      z.e[pr][0] = __builtin_amdgcn_exp2f(T[kb][r]);
      z.e[pr][1] = __builtin_amdgcn_exp2f(T[kb][r + 1]);
      pin(z.e[pr][0]);
      pin(z.e[pr][1]);
    };
    auto soft_b_pack = [&](int pr, SoftB& z) {
      const int kb = pr >> 3, r = 2 * (pr & 7);
      z.pk[pr] = pack_bf16x2(z.e[pr][0], z.e[pr][1]);
      pin(z.pk[pr]);
      pf[2 * kb + (r >> 3)][(r & 7) >> 1] = z.pk[pr];
    };
    auto soft_b_sum = [&](int pr, SoftB& z) {
      // row sum of the bf16 weights the P.V product actually applies
      z.rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, z.pk[pr]),
                                             __builtin_bit_cast(bf16x2_t, 0x3f803f80u), z.rs,
                                             false);
      pin(z.rs);   // summed in its slot, not sunk to the end of the step
    };
    auto soft_b = [&](f32x16_t (&T)[NKB], int x, SoftB& z) {
#pragma unroll
      for (int i = 0; i < PPS; ++i) {
        soft_b_exp(T, x * PPS + i, z);
        if (x >= 1) soft_b_pack((x - 1) * PPS + i, z);
        if (x >= 2) soft_b_sum((x - 2) * PPS + i, z);
      }
    };
    auto soft_b_drain = [&](SoftB& z) {
#pragma unroll
      for (int i = 0; i < PPS; ++i) soft_b_pack((NSLOT - 1) * PPS + i, z);
#pragma unroll
      for (int i = 0; i < 2 * PPS; ++i) soft_b_sum((NSLOT - 2) * PPS + i, z);
    };

    // ---- phase 1: S_next = K Q^T (when `next`) beside the exponentials of T
    auto phase1 = [&](bool next, f32x16_t (&Snext)[NKB], f32x16_t (&T)[NKB],
                      const unsigned char* kl, unsigned char* kdst, unsigned char* vdst) {
      __amdgpu_buffer_rsrc_t rk, rv;
      if (next) {
        rk = kv_rsrc(curK, false);
        rv = kv_rsrc(curV, true);
      }
      SoftB z;
      z.rs = 0.f;
      constexpr int AH = 2;  // K operands read this many slots ahead
      u32x4_t opnd[AH + 1];
      auto rdk = [&](int x) {
        return *reinterpret_cast<const u32x4_t*>(kl + kad[x % NDS] + (x / NDS) * 32 * RB);
      };
      if (next) {
#pragma unroll
        for (int x = 0; x < AH; ++x) opnd[x] = rdk(x);
      }
      constexpr int NDMA = 2 * KV_DMA;
#pragma unroll
      for (int x = 0; x < NSLOT; ++x) {
        if (next) {
          if (x + AH < NSLOT) opnd[(x + AH) % (AH + 1)] = rdk(x + AH);
          const int kb = x / NDS, s = x % NDS;
          Snext[kb] = mfma32x32x16(opnd[x % (AH + 1)], qf[s], s == 0 ? f32x16_t{} : Snext[kb]);
          // this slot's share of the next tiles' loads
#pragma unroll
          for (int d = 0; d < NDMA; ++d) {
            if (d * NSLOT / NDMA != x) continue;
            if (d < KV_DMA) dma_kv(rk, kdst, d);
            else dma_kv(rv, vdst, d - KV_DMA);
          }
        }
        soft_b(T, x, z);
        __builtin_amdgcn_sched_barrier(0);
      }
      soft_b_drain(z);
      lsum += z.rs;
      pin(lsum);
    };

    // ---- phase 2: O += P V beside the first softmax half of S_next
    auto phase2 = [&](bool next, f32x16_t (&Snext)[NKB], const unsigned char* vl) {
      constexpr int AH = 2;
      s16x4_t opnd[AH + 1][2];
      auto rd = [&](int y) {
        const int t = y / NDB, db = y % NDB;
        opnd[y % (AH + 1)][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(vl + vad[db][0] + t * 16 * RB));
        opnd[y % (AH + 1)][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(vl + vad[db][1] + t * 16 * RB));
      };
#pragma unroll
      for (int y = 0; y < AH; ++y) rd(y);
      SoftA z;
#pragma unroll
      for (int y = 0; y < NSLOT2; ++y) {
        if (y + AH < NSLOT2) rd(y + AH);
        const int t = y / NDB, db = y % NDB;
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, opnd[y % (AH + 1)][0]);
        const u32x2_t hi = __builtin_bit_cast(u32x2_t, opnd[y % (AH + 1)][1]);
        oacc[db] = mfma32x32x16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf[t], oacc[db]);
        if (next) {
#pragma unroll
          for (int k = 0; k < NSTAGE_A; ++k)
            if (k * NSLOT2 / NSTAGE_A == y) soft_a(Snext, k, z);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    auto rescale_o = [&]() {
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
    };

    // ---- first tile: scores and softmax half, with the loads of V of the
    // first tile and K of the second spread between the products
    if (n_g > 0) {
      const auto rv = kv_rsrc(cur0, true);
      const auto rk1 = kv_rsrc(curV, false);   // zero-length past the last tile
      constexpr int NDMA0 = 2 * KV_DMA;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          const int x = kb * NDS + s;
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&k_lds0[0][0] + kad[s] +
                                                             kb * 32 * RB);
          sA[kb] = mfma32x32x16(a, qf[s], s == 0 ? f32x16_t{} : sA[kb]);
#pragma unroll
          for (int d = 0; d < NDMA0; ++d) {
            if (d * NSLOT / NDMA0 != x) continue;
            if (d < KV_DMA) dma_kv(rv, v_lds0[grp], d);
            else dma_kv(rk1, k_lds1[grp], d - KV_DMA);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      const TileInfo ti = tile_info(cur0);
      if (!ti.full) apply_mask(sA, tile_bits(ti));
      SoftA z;
#pragma unroll
      for (int k = 0; k < NSTAGE_A; ++k) soft_a(sA, k, z);
    }
    // V of the first tile and K of the second have landed, and every wave
    // is done with the first K buffer before it is refilled
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();

    // ---- key loop: step u computes S of tile u+1 and O += P_u V_u; this
    // group's tiles are grp + KSPLIT u.  Steps with a next tile run one
    // straight-line body (only the boundary mask and the rare rescale
    // branch); the last step and the idle steps of a group with one tile
    // fewer follow the loop.
    auto step_next = [&](f32x16_t (&T)[NKB], f32x16_t (&Sn)[NKB], const unsigned char* kl,
                         const unsigned char* vl, unsigned char* kdst, unsigned char* vdst) {
      // loads: K of the tile after next (curK), V of the next (curV)
      phase1(true, Sn, T, kl, kdst, vdst);
      const TileInfo ti = tile_info(curV);
      if (!ti.full) apply_mask(Sn, tile_bits(ti));
      phase2(true, Sn, vl);
      rescale_o();
      curV = curK;
      curK = cur_next(curK);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads landed
      __syncthreads();
    };
    auto step_last = [&](f32x16_t (&T)[NKB], f32x16_t (&Sn)[NKB], const unsigned char* vl) {
      phase1(false, Sn, T, nullptr, nullptr, nullptr);
      phase2(false, Sn, vl);
      __syncthreads();
    };
    // unrolled by two: even steps read sA / k_lds1 / v_lds0, odd steps the
    // others, so every buffer reference is a fixed object (the operand reads
    // take the array base; their offsets hold the key group's slot)
    const int n_next = n_g - 1;   // steps with a next tile
    int u = 0;
    for (; u + 1 < n_next; u += 2) {
      step_next(sA, sB, &k_lds1[0][0], &v_lds0[0][0], k_lds0[grp], v_lds1[grp]);
      step_next(sB, sA, &k_lds0[0][0], &v_lds1[0][0], k_lds1[grp], v_lds0[grp]);
    }
    if (u < n_next) {
      step_next(sA, sB, &k_lds1[0][0], &v_lds0[0][0], k_lds0[grp], v_lds1[grp]);
      ++u;
    }
    if (n_g > 0) {
      if ((u & 1) == 0) step_last(sA, sB, &v_lds0[0][0]);
      else step_last(sB, sA, &v_lds1[0][0]);
    }
    for (int w = max(n_g, 0); w < n_steps; ++w) __syncthreads();

    float ltot = pair_sum(lsum);
    // the epilogue's per-lane addresses come from an opaque copy of the lane
    // id: computed here, instead of being hoisted to the kernel start into
    // registers the key loop has to spill (whose reloads then wait for every
    // outstanding store)
    uint32_t eln = (uint32_t)lane;
    asm volatile("" : "+v"(eln));
    const uint32_t ecol = eln & 31u, ehalf = eln >> 5;
    const int eqi = iw + (int)ecol;
    // ACC: the accumulator's LSE of this lane's row, read (and waited for)
    // before the exchange barrier, after which group 0 may overwrite it
    const size_t li = (size_t)head * p.l_q + min(eqi, last_row);
    float la = 0.f;
    if constexpr (ACC) {
      la = p.lse_acc[li];
      asm volatile("" : "+v"(la));
    }

    // ---- the rows' final (O, m, l) and where they go.  KSPLIT = 2: the two
    // key groups merge through LDS; group 0 then finishes head dims
    // [0, D/2), group 1 [D/2, D).  KSPLIT = 1: every wave finishes its rows.
    constexpr int NDBH = KSPLIT == 2 ? NDB / 2 : NDB;   // 32-dim blocks finished
    const int db0 = KSPLIT == 2 ? grp * NDBH : 0;       // first of them
    // the blocks this wave finishes, picked by value (a uniform select), so
    // that every register array keeps compile-time indices
    f32x16_t fin[NDBH];
    if constexpr (KSPLIT == 2) {
      // exchange: each wave stores the dim blocks it hands over (float4 f of
      // lane l at (f, wave, l)) in the V buffers and its (m, l) in the Q
      // buffer; the partner wave (same rows, other group) reads them
      f32x16_t give[NDBH];
#pragma unroll
      for (int i = 0; i < NDBH; ++i) {
        fin[i] = grp == 0 ? oacc[i] : oacc[NDBH + i];
        give[i] = grp == 0 ? oacc[NDBH + i] : oacc[i];
      }
      constexpr int NF = 4 * NDBH;
      static_assert(kWaves * (NF / 2) * 64 * 16 <= KSPLIT * TILE, "exchange fits");
      // float4 f of every wave: the first NF / 2 in one V buffer, the rest
      // in the other
      auto xo = [&](int f, int w) -> float4& {
        float4* base = reinterpret_cast<float4*>(f < NF / 2 ? &v_lds0[0][0] : &v_lds1[0][0]);
        return base[((f % (NF / 2)) * kWaves + w) * 64 + eln];
      };
      float2* xml = xml_lds;
      const int partner = (wave_all + WPG) % kWaves;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int i = f / 4, r = 4 * (f % 4);
        xo(f, wave_all) = make_float4(give[i][r], give[i][r + 1], give[i][r + 2], give[i][r + 3]);
      }
      xml[wave_all * 64 + eln] = make_float2(m, ltot);
      __syncthreads();
      const float2 ml = xml[partner * 64 + eln];
      // group 0's and group 1's (m, l), combined in one fixed order so both
      // groups get the same merged values
      const float m0 = grp == 0 ? m : ml.x, l0 = grp == 0 ? ltot : ml.y;
      const float m1 = grp == 0 ? ml.x : m, l1 = grp == 0 ? ml.y : ltot;
      const float mm = fmaxf(m0, m1);
      const float w0 = (m0 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
      const float w1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      const float wown = grp == 0 ? w0 : w1, woth = grp == 0 ? w1 : w0;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int i = f / 4, r = 4 * (f % 4);
        const float4 x = xo(f, partner);
        fin[i][r] = fin[i][r] * wown + x.x * woth;
        fin[i][r + 1] = fin[i][r + 1] * wown + x.y * woth;
        fin[i][r + 2] = fin[i][r + 2] * wown + x.z * woth;
        fin[i][r + 3] = fin[i][r + 3] * wown + x.w * woth;
      }
      ltot = l0 * w0 + l1 * w1;
      m = mm;
    } else {
#pragma unroll
      for (int i = 0; i < NDBH; ++i) fin[i] = oacc[i];
    }

    const float muse = (m == kNegInf) ? 0.f : m;
    const float lse_b = ltot > 0.f ? (muse + __log2f(ltot)) * kLn2 : kNegInf;
    // this wave's staging slice: 32 rows of the finished dims, in the K
    // buffers (KSPLIT = 2: waves 0-3 in one, 4-7 in the other; the exchange
    // used the V buffers) or two waves to each K and V buffer (KSPLIT = 1);
    // all are free since the loop ended
    unsigned char* stage;
    if constexpr (KSPLIT == 2) {
      static_assert(4 * 32 * RB <= KSPLIT * TILE, "staging fits");
      stage = (wave_all < 4 ? &k_lds0[0][0] : &k_lds1[0][0]) + (wave_all % 4) * 32 * RB;
    } else {
      static_assert(2 * 32 * RB <= TILE, "staging fits");
      const int w2 = wave_all / 2;
      stage = (w2 == 0 ? &k_lds0[0][0] : w2 == 1 ? &k_lds1[0][0] : w2 == 2 ? &v_lds0[0][0]
                                                                           : &v_lds1[0][0]) +
              (wave_all % 2) * 32 * RB;
    }
    if constexpr (ACC) {
      // merge (O / l, LSE) into the accumulator rows (log1p form, the -inf
      // guards of attn_merge: 0 keep, 1 replace, 2 weighted sum, 3 clear);
      // the finished dims pass through LDS in fp32, 16 rows per round, so
      // every accumulator access is a contiguous run of the row
      int mode = la == kNegInf ? 3 : 0;
      float wa = 0.f, wb = 0.f, lnew = la;
      if (lse_b != kNegInf) {
        if (la == kNegInf) {
          mode = 1;
          wb = 1.f / ltot;
          lnew = lse_b;
        } else {
          mode = 2;
          const float mx = fmaxf(la, lse_b), mn = fminf(la, lse_b);
          lnew = mx + log1pf(expf(mn - mx));
          wa = expf(la - lnew);
          wb = expf(lse_b - lnew) / ltot;
        }
      }
      constexpr int CH = NDBH * 8;   // 16-byte fp32 chunks of the finished dims
      float* fst = reinterpret_cast<float*>(stage);
      static_assert(16 * CH * 16 <= 32 * RB, "16 fp32 rows fit the slice");
#pragma unroll
      for (int round = 0; round < 2; ++round) {
        if ((ecol >> 4) == (uint32_t)round) {
          const uint32_t row = ecol & 15u;
#pragma unroll
          for (int i = 0; i < NDBH; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const uint32_t cc = (uint32_t)(8 * i + 2 * r4) + ehalf;
              const f32x4_t x = {fin[i][4 * r4] * wb, fin[i][4 * r4 + 1] * wb,
                                 fin[i][4 * r4 + 2] * wb, fin[i][4 * r4 + 3] * wb};
              *reinterpret_cast<f32x4_t*>(fst + row * (4 * CH) + 4 * (cc ^ (2u * row % CH))) = x;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int it = 0; it < 16 * CH / 64; ++it) {
          const int k = it * 64 + (int)eln;
          const int rr = k / CH, cc = k % CH;
          const int src = 16 * round + rr;  // the lane that holds this row
          const int rmode = __shfl(mode, src);
          const float rwa = __shfl(wa, src);
          const int i = iw + src;
          const f32x4_t x =
              *reinterpret_cast<const f32x4_t*>(fst + rr * (4 * CH) + 4 * (cc ^ (2 * rr % CH)));
          if (i <= last_row && rmode != 0) {
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(
                p.acc + ((size_t)b * p.l_q + i) * q_row + (size_t)hq * D + 32 * db0 + 4 * cc);
            *dst = rmode == 1 ? x : rmode == 3 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : *dst * rwa + x;
          }
        }
        // the next round overwrites what this round read
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      // both groups read the accumulator's LSE before the exchange barrier;
      // only group 0 writes the new one
      if (grp == 0 && ehalf == 0 && eqi <= last_row && (mode == 1 || mode == 2))
        p.lse_acc[li] = lnew;
    } else {
      // normalise and stage the 32 rows (bf16, 16-byte chunks swizzled by row
      // like the tiles), then store contiguous runs of every row
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
      for (int i = 0; i < NDBH; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2_t w;
          w[0] = pack_bf16x2(fin[i][4 * r4] * inv, fin[i][4 * r4 + 1] * inv);
          w[1] = pack_bf16x2(fin[i][4 * r4 + 2] * inv, fin[i][4 * r4 + 3] * inv);
          const uint32_t cc = (uint32_t)(4 * (db0 + i) + r4) ^ chunk_swz<D>(ecol);
          *reinterpret_cast<u32x2_t*>(stage + ecol * RB + cc * 16 + 8 * ehalf) = w;
        }
      // the wave reads back what its own lanes wrote: LDS operations of one
      // wave complete in order once counted down
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      constexpr int CPH = NDBH * 4;   // 16-byte chunks finished per row
      constexpr int RPI = 64 / CPH;   // rows per store instruction
      constexpr int NST = 32 / RPI;   // store instructions
      // every read first, then the stores (no wait between stores)
      u32x4_t val[NST];
      const uint32_t c = 4u * (uint32_t)db0 + eln % CPH;
#pragma unroll
      for (int x = 0; x < NST; ++x) {
        const uint32_t r = (uint32_t)(x * RPI) + eln / CPH;
        val[x] = *reinterpret_cast<const u32x4_t*>(stage + r * RB +
                                                   (c ^ chunk_swz<D>(r)) * 16);
      }
      uint16_t* const obase = p.o + ((size_t)b * p.l_q + iw) * q_row + (size_t)hq * D;
#pragma unroll
      for (int x = 0; x < NST; ++x) {
        const uint32_t r = (uint32_t)(x * RPI) + eln / CPH;
        if (iw + (int)r <= last_row)
          __builtin_nontemporal_store(val[x],
                                      reinterpret_cast<u32x4_t*>(obase + (size_t)r * q_row + 8 * c));
      }
      if (grp == 0 && ehalf == 0 && eqi <= last_row) p.lse[(size_t)head * p.l_q + eqi] = lse_b;
    }
  };

  const int n_tiles = p.pairs ? (unit == p.n_qtiles - 1 - unit ? 1 : 2) : 1;
  for (int ti = 0; ti < n_tiles; ++ti) {
    // pairing: the shorter tile r first, then n_qtiles-1-r; under a causal
    // mask the longer one then finds the shorter one's keys in L2
    const int tile = p.pairs ? (ti == 1 ? p.n_qtiles - 1 - unit : unit) : unit;
    // the previous tile's exchange and staging use buffers this tile's
    // first loads overwrite
    if (ti > 0) __syncthreads();
    fwd_tile(tile);
  }
}

// Schedules: KSPLIT = 2 (128-row q tiles, two key groups) with or without
// pairing of q tiles r and n_qtiles-1-r, or KSPLIT = 1 (256-row q tiles).
// One workgroup per CU; the choice minimises max(longest workgroup, total /
// CUs) in units of one step (eight waves x 32 rows x 64 keys), the
// single-group step charged a little less (half the K/V loads per step) and
// pairing preferred on a tie (the long tile finds the short one's keys in
// L2, and no second round of workgroups starts cold).
struct PipeSchedule {
  int ksplit;
  int pairs;
};

constexpr int kCUs = 256;

// The pipelined loop pays more per q tile (a deeper prologue, the two-phase
// fill and drain) than the one-phase kernel of fwd.hip and gains per key
// tile: it is the better kernel once q tiles see this many key tiles on
// average (measured on gfx950: 16-17 per 128-row q tile, the causal
// 2 x 2048-token and the 1024-key ring step workloads, already favour it by
// 3-10%; the 256-key window's 6-7 favour the one-phase kernel by 40%).
constexpr int kPipeMinTiles = 12;

int tiles_of(const PipeParams& p, int rows, int tile) {
  const int i0 = tile * rows;
  const int il = std::min(i0 + rows, p.l_q) - 1;
  int t = 0;
  for (int c = 0; c < p.n_chunks; ++c) {
    const long long jlo = std::max(0LL, (long long)i0 + p.ch[c].dlo);
    const long long jhi = std::min((long long)p.ch[c].l_k - 1, (long long)il + p.ch[c].dhi);
    if (jlo <= jhi) t += (int)(jhi / kBN - jlo / kBN + 1);
  }
  return t;
}

PipeSchedule pick_pipe_schedule(const PipeParams& p, bool allow_ks1) {
  const double heads = p.n_heads;
  double best = 1e300;
  PipeSchedule out{2, 0};
  for (int ks = 2; ks >= 1; --ks) {
    if (ks == 1 && !allow_ks1) continue;
    const int rows = 32 * (kWaves / ks);
    const int nt = (p.l_q + rows - 1) / rows;
    for (int pr = 0; pr <= 1; ++pr) {
      long long mx = 0, sum = 0;
      const int units = pr ? (nt + 1) / 2 : nt;
      for (int r = 0; r < units; ++r) {
        long long len = (tiles_of(p, rows, r) + ks - 1) / ks;
        if (pr && nt - 1 - r != r) len += (tiles_of(p, rows, nt - 1 - r) + ks - 1) / ks;
        mx = std::max(mx, len);
        sum += len;
      }
      const double cost =
          (ks == 1 ? 0.97 : 1.0) * (pr ? 0.99 : 1.0) * std::max((double)mx, (double)sum * heads / kCUs);
      if (cost < best) {
        best = cost;
        out = PipeSchedule{ks, pr};
      }
    }
  }
  return out;
}

template <int D, int KS, bool ACC, bool MULTI>
void launch_one(const PipeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_pipe_kernel<D, KS, ACC, MULTI>), grid, dim3(kThreads), 0, stream, p);
}

template <bool ACC, bool MULTI>
void launch_d(const PipeParams& p, int d, int ks, dim3 grid, hipStream_t stream) {
  if (d == 128) {
    if (ks == 2) launch_one<128, 2, ACC, MULTI>(p, grid, stream);
    else launch_one<128, 1, ACC, MULTI>(p, grid, stream);
  } else {
    if (ks == 2) launch_one<64, 2, ACC, MULTI>(p, grid, stream);
    else launch_one<64, 1, ACC, MULTI>(p, grid, stream);
  }
}

}  // namespace

hipError_t launch_fwd_pipe(const void* q, const FwdChunk* chunks, int n_chunks, void* out,
                           float* lse, const AttnShape& s, hipStream_t stream, float* acc,
                           float* lse_acc, int force_ksplit) {
  PipeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.acc = acc;
  p.lse_acc = lse_acc;
  for (int c = 0; c < kMaxChunks; ++c) p.ch[c] = c < n_chunks ? chunks[c] : chunks[0];
  p.n_chunks = n_chunks;
  p.l_q = s.l_q;
  p.h = s.h;
  p.h_kv = s.h_kv;
  p.grp = s.h / s.h_kv;
  p.n_heads = s.n * s.h;
  p.xcd_groups = ((s.n * s.h_kv) % 8 == 0) ? 1 : 0;
  p.reverse = s.causal ? 1 : 0;
  p.c = (s.scale == 0.f ? 1.f : fabsf(s.scale)) * kLog2e;
  p.q_and = s.scale == 0.f ? 0u : 0xffffffffu;
  p.q_xor = s.scale < 0.f ? 0x80008000u : 0u;
  // the 256-row Q tile is addressed with 32-bit offsets from its first row
  const bool allow_ks1 = 256LL * s.h * s.d * 2 < (1LL << 31);
  PipeSchedule sch = pick_pipe_schedule(p, allow_ks1);
  if (force_ksplit == 2 || (force_ksplit == 1 && allow_ks1)) {
    sch.ksplit = force_ksplit;
    sch.pairs = 0;
  }
  const int rows = 32 * (kWaves / sch.ksplit);
  p.n_qtiles = (s.l_q + rows - 1) / rows;
  p.pairs = sch.pairs;
  p.n_units = p.pairs ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const dim3 grid((unsigned)p.n_units * (unsigned)p.n_heads);
  const bool multi = n_chunks > 1;
  if (acc == nullptr) {
    if (multi) launch_d<false, true>(p, s.d, sch.ksplit, grid, stream);
    else launch_d<false, false>(p, s.d, sch.ksplit, grid, stream);
  } else {
    // a fused step always covers one chunk
    if (multi) return hipErrorInvalidValue;
    launch_d<true, false>(p, s.d, sch.ksplit, grid, stream);
  }
  return hipGetLastError();
}

const char* fwd_pipe_kernel_name(const FwdChunk* chunks, int n_chunks, const AttnShape& s,
                                 bool acc) {
  PipeParams p;
  for (int c = 0; c < kMaxChunks; ++c) p.ch[c] = c < n_chunks ? chunks[c] : chunks[0];
  p.n_chunks = n_chunks;
  p.l_q = s.l_q;
  p.n_heads = s.n * s.h;
  const PipeSchedule sch = pick_pipe_schedule(p, 256LL * s.h * s.d * 2 < (1LL << 31));
  static const char* const names[2][2][3] = {
      {{"fwd_pipe_kernel<64, 1, false, false>", "fwd_pipe_kernel<64, 1, false, true>",
        "fwd_pipe_kernel<64, 1, true, false>"},
       {"fwd_pipe_kernel<64, 2, false, false>", "fwd_pipe_kernel<64, 2, false, true>",
        "fwd_pipe_kernel<64, 2, true, false>"}},
      {{"fwd_pipe_kernel<128, 1, false, false>", "fwd_pipe_kernel<128, 1, false, true>",
        "fwd_pipe_kernel<128, 1, true, false>"},
       {"fwd_pipe_kernel<128, 2, false, false>", "fwd_pipe_kernel<128, 2, false, true>",
        "fwd_pipe_kernel<128, 2, true, false>"}}};
  const int form = acc ? 2 : (n_chunks > 1 ? 1 : 0);
  return names[s.d == 128 ? 1 : 0][sch.ksplit == 2 ? 1 : 0][form];
}

bool fwd_pipe_preferred(const FwdChunk* chunks, int n_chunks, const AttnShape& s) {
  // mean key tiles per 128-row q tile over the chunks
  PipeParams p;
  for (int c = 0; c < kMaxChunks; ++c) p.ch[c] = c < n_chunks ? chunks[c] : chunks[0];
  p.n_chunks = n_chunks;
  p.l_q = s.l_q;
  const int nt = (s.l_q + 127) / 128;
  long long sum = 0;
  for (int t = 0; t < nt; ++t) sum += tiles_of(p, 128, t);
  return sum >= (long long)kPipeMinTiles * nt;
}

}  // namespace bea
