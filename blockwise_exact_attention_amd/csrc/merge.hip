// The (O, LSE) merge of partial attention results and the ring accumulator's
// set-up and final cast, for gfx950.  All three are elementwise and bound by
// HBM bandwidth.
//
// Sources: "flash_sharding.py" (flash_attn_jax), ring_fwd - accumulator
// starts at O = 0 (fp32) and LSE = -inf; each chunk's O is upcast to fp32 and
// merged as lse = max + log1p(exp(min - max)),
// o = o1 exp(lse1 - lse) + o2 exp(lse2 - lse); the result is cast back to the
// query dtype at the end.  "picotron/parallel/context_parallel.py",
// update_out_and_lse - the same merge in sigmoid form, and the first block
// simply becomes the accumulator (here: whenever the accumulator's LSE is
// -inf).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace bea {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeMaxRows = 256;
constexpr int kMergeElems = 2048;  // elements per block on the vector path
constexpr int kMergeVec = kMergeElems / (4 * kMergeThreads);  // float4 per thread

// Row weights: mode 0 keep the accumulator, 1 take the block, 2 weighted
// sum, 3 clear the row (both sides empty: the merged row is the empty
// result O = 0, LSE = -inf, whatever the accumulator held).  Computed once
// per row by one thread and shared through LDS; that thread also writes the
// row's new LSE (no other thread reads it).
__device__ __forceinline__ void merge_row_weights(float* __restrict__ lse_acc,
                                                  const float* __restrict__ lse_blk,
                                                  int l, int h, long long row,
                                                  int& mode, float& wa, float& wb) {
  // rows are ordered (b, i, hq) like O; the LSE of that row sits at [b, hq, i]
  const long long bi = row / h;
  const int hq = (int)(row - bi * h);
  const long long b = bi / l;
  const int i = (int)(bi - b * l);
  const size_t li = ((size_t)b * h + hq) * l + i;
  const float a = lse_acc[li];
  const float bb = lse_blk[li];
  wa = 0.f;
  wb = 0.f;
  if (bb == kNegInf) {
    mode = a == kNegInf ? 3 : 0;
  } else if (a == kNegInf) {
    mode = 1;
    lse_acc[li] = bb;
  } else {
    mode = 2;
    const float mx = fmaxf(a, bb);
    const float mn = fminf(a, bb);
    const float lse = mx + log1pf(expf(mn - mx));
    wa = expf(a - lse);
    wb = expf(bb - lse);
    lse_acc[li] = lse;
  }
}

// Vector path (d % 4 == 0, 2048 / d rows per block): a block covers
// consecutive query rows i0 .. i0 + R - 1 of one (batch, head), so its LSE
// reads are contiguous; its O rows are R rows h*d apart, each row contiguous.
// Every thread issues its data loads (the block's values and, speculatively,
// the accumulator's) before the row weights are known, so a block pays one
// memory round trip, not two.  The O data is touched once per merge: its
// loads and stores carry the nontemporal hint (streamed past the caches;
// measured on gfx950 from HBM: 11.3 -> 9.6 us for a 42 MB merge).
// One block of the vector path: rows i0 .. i0 + R - 1 of (batch b, head hq),
// bh = b * h + hq.
template <bool BLK_BF16>
__device__ __forceinline__ void merge_vec_block(
    float* __restrict__ acc, float* __restrict__ lse_acc, const void* __restrict__ blk,
    const float* __restrict__ lse_blk, int l, int h, int d, size_t bh, size_t b, int hq,
    int i0, float* s_wa, float* s_wb, int* s_mode) {
  const int R = kMergeElems / d;
  const int nr = min(R, l - i0);
  const int tid = threadIdx.x;
  const size_t row_stride = (size_t)h * d;
  const size_t base = ((size_t)b * l + i0) * row_stride + (size_t)hq * d;

  // the row's two LSE values first: their round trip decides the weights
  float la = kNegInf, lb = kNegInf;
  const size_t li = (size_t)bh * l + i0 + tid;
  if (tid < nr) {
    la = lse_acc[li];
    lb = lse_blk[li];
  }
  f32x4_t av[kMergeVec], bv[kMergeVec];
#pragma unroll
  for (int v = 0; v < kMergeVec; ++v) {
    const int e = (v * kMergeThreads + tid) * 4;
    const int rr = e / d;
    if (rr < nr) {
      const size_t off = base + (size_t)rr * row_stride + (e - rr * d);
      if (BLK_BF16) {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
            static_cast<const uint16_t*>(blk) + off));
        bv[v] = f32x4_t{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      } else {
        bv[v] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(static_cast<const float*>(blk) + off));
      }
      av[v] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(acc + off));
    }
  }
  if (tid < nr) {
    const float a = la;
    const float bb = lb;
    int mode = 2;
    float wa = 0.f, wb = 0.f;
    if (bb == kNegInf) {
      mode = a == kNegInf ? 3 : 0;
    } else if (a == kNegInf) {
      mode = 1;
      lse_acc[li] = bb;
    } else {
      const float mx = fmaxf(a, bb);
      const float mn = fminf(a, bb);
      const float lse = mx + log1pf(expf(mn - mx));
      wa = expf(a - lse);
      wb = expf(bb - lse);
      lse_acc[li] = lse;
    }
    s_mode[tid] = mode;
    s_wa[tid] = wa;
    s_wb[tid] = wb;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < kMergeVec; ++v) {
    const int e = (v * kMergeThreads + tid) * 4;
    const int rr = e / d;
    if (rr >= nr) continue;
    const int mode = s_mode[rr];
    const size_t off = base + (size_t)rr * row_stride + (e - rr * d);
    // a row whose accumulator LSE is -inf takes the block as is, or zeros
    // when the block row is empty too (select, never a multiply, so
    // whatever the accumulator held cannot leak)
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(acc + off);
    if (mode == 1)
      __builtin_nontemporal_store(bv[v], dst);
    else if (mode == 3)
      __builtin_nontemporal_store(f32x4_t{0.f, 0.f, 0.f, 0.f}, dst);
    else if (mode == 2)
      __builtin_nontemporal_store(av[v] * s_wa[rr] + bv[v] * s_wb[rr], dst);
  }
}

// WALK: the grid is capped and walks the blocks in several passes (shapes
// beyond 2^20 blocks); otherwise every block merges its own rows once.
template <bool BLK_BF16, bool WALK>
__global__ __launch_bounds__(kMergeThreads) void merge_vec_kernel(
    float* __restrict__ acc, float* __restrict__ lse_acc,
    const void* __restrict__ blk, const float* __restrict__ lse_blk, int l,
    int h, int d, int iblocks, long long nblocks) {
  __shared__ float s_wa[kMergeMaxRows];
  __shared__ float s_wb[kMergeMaxRows];
  __shared__ int s_mode[kMergeMaxRows];
  const int R = kMergeElems / d;
  if (!WALK) {
    const int bh = blockIdx.x / iblocks;       // b * h + hq
    const int i0 = (blockIdx.x - bh * iblocks) * R;
    const int b = bh / h;
    const int hq = bh - b * h;
    merge_vec_block<BLK_BF16>(acc, lse_acc, blk, lse_blk, l, h, d, (size_t)bh, (size_t)b, hq,
                              i0, s_wa, s_wb, s_mode);
    return;
  }
  for (long long vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
    const long long bh = vb / iblocks;
    const int i0 = (int)(vb - bh * iblocks) * R;
    const long long b = bh / h;
    const int hq = (int)(bh - b * h);
    merge_vec_block<BLK_BF16>(acc, lse_acc, blk, lse_blk, l, h, d, (size_t)bh, (size_t)b, hq,
                              i0, s_wa, s_wb, s_mode);
    __syncthreads();   // the next block's weights overwrite s_mode, s_wa, s_wb
  }
}

// Scalar path for any other d: a block covers up to 1024 / d rows.
template <bool BLK_BF16>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    float* __restrict__ acc, float* __restrict__ lse_acc,
    const void* __restrict__ blk, const float* __restrict__ lse_blk, int l,
    int h, int d, long long rows_total, int rows_per_block, long long nblocks) {
  __shared__ float s_wa[kMergeMaxRows];
  __shared__ float s_wb[kMergeMaxRows];
  __shared__ int s_mode[kMergeMaxRows];

  for (long long vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
  const long long r0 = vb * rows_per_block;
  const int nr = (int)min((long long)rows_per_block, rows_total - r0);
  const int tid = threadIdx.x;
  if (tid < nr) {
    int mode;
    float wa, wb;
    merge_row_weights(lse_acc, lse_blk, l, h, r0 + tid, mode, wa, wb);
    s_mode[tid] = mode;
    s_wa[tid] = wa;
    s_wb[tid] = wb;
  }
  __syncthreads();

  const size_t e0 = (size_t)r0 * d;
  const int ne = nr * d;
  for (int e = tid; e < ne; e += kMergeThreads) {
    const int rr = e / d;
    const int mode = s_mode[rr];
    if (mode == 0) continue;
    if (mode == 3) {
      acc[e0 + e] = 0.f;
      continue;
    }
    const float bv = BLK_BF16
        ? bf16_lo(static_cast<const uint16_t*>(blk)[e0 + e])
        : static_cast<const float*>(blk)[e0 + e];
    acc[e0 + e] = (mode == 1) ? bv : acc[e0 + e] * s_wa[rr] + bv * s_wb[rr];
  }
  __syncthreads();
  }
}

// Merge of an empty block (every row's LSE -inf, e.g. a chunk with no keys)
// into the accumulator: rows at -inf are cleared to O = 0, all others stay.
// One block per 256 rows; row r of [n, l, h] order (b, i, hq).
__global__ __launch_bounds__(256) void acc_clear_empty_kernel(float* __restrict__ acc,
                                                              const float* __restrict__ lse_acc,
                                                              int l, int h, int d,
                                                              long long rows) {
  __shared__ int s_clear[256];
  for (long long r0 = (long long)blockIdx.x * 256; r0 < rows; r0 += (long long)gridDim.x * 256) {
  const int nr = (int)min(256LL, rows - r0);
  const int tid = threadIdx.x;
  if (tid < nr) {
    const long long row = r0 + tid;
    const long long bi = row / h;
    const int hq = (int)(row - bi * h);
    const long long b = bi / l;
    const int i = (int)(bi - b * l);
    s_clear[tid] = lse_acc[((size_t)b * h + hq) * l + i] == kNegInf;
  }
  __syncthreads();
  const size_t e0 = (size_t)r0 * d;
  const int ne = nr * d;
  for (int e = tid; e < ne; e += 256)
    if (s_clear[e / d]) acc[e0 + e] = 0.f;
  __syncthreads();
  }
}

// 16-byte stores where the accumulator is 16-byte aligned (n4 = n_acc / 4),
// 4-byte stores for the rest.
__global__ __launch_bounds__(256) void acc_init_kernel(float* __restrict__ acc,
                                                       float* __restrict__ lse,
                                                       long long n_acc,
                                                       long long n4,
                                                       long long n_lse) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (long long e = t; e < n4; e += stride)
    reinterpret_cast<f32x4_t*>(acc)[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (long long e = n4 * 4 + t; e < n_acc; e += stride) acc[e] = 0.f;
  for (long long e = t; e < n_lse; e += stride) lse[e] = kNegInf;
}

template <bool BF16>
__global__ __launch_bounds__(256) void acc_cast_kernel(const float* __restrict__ acc,
                                                       void* __restrict__ out,
                                                       long long n_elem) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long n4 = n_elem / 4;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += stride) {
    const f32x4_t x = reinterpret_cast<const f32x4_t*>(acc)[e];
    if (BF16) {
      u32x2_t w;
      w[0] = pack_bf16x2(x[0], x[1]);
      w[1] = pack_bf16x2(x[2], x[3]);
      reinterpret_cast<u32x2_t*>(out)[e] = w;
    } else {
      reinterpret_cast<f32x4_t*>(out)[e] = x;
    }
  }
  for (long long e = n4 * 4 + (long long)blockIdx.x * blockDim.x + threadIdx.x;
       e < n_elem; e += stride) {
    if (BF16) {
      const uint32_t w = pack_bf16x2(acc[e], 0.f);
      static_cast<uint16_t*>(out)[e] = (uint16_t)(w & 0xffffu);
    } else {
      static_cast<float*>(out)[e] = acc[e];
    }
  }
}

// A plain read-and-write stream of n4 16-byte words (nontemporal loads and
// stores, one word per thread): what an elementwise kernel's HBM traffic can
// reach on this GPU, the reference the merge is measured against.
__global__ __launch_bounds__(256) void hbm_copy_kernel(const f32x4_t* __restrict__ src,
                                                       f32x4_t* __restrict__ dst,
                                                       long long n4) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n4;
       e += (long long)gridDim.x * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + e), dst + e);
}

}  // namespace

// A grid of at most 2^20 blocks: launches count work-items in 32 bits, so the
// elementwise kernels walk larger block counts in several passes.
unsigned capped_grid(long long blocks) {
  return (unsigned)std::max(1LL, std::min(blocks, 1LL << 20));
}

namespace {

unsigned grid_for(long long work, int per_block) {
  long long g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_merge(float* out_acc, float* lse_acc, const void* out_blk,
                        const float* lse_blk, int n, int l, int h, int d,
                        bool blk_bf16, hipStream_t stream) {
  const long long rows = (long long)n * l * h;
  if (d % 4 == 0 && d <= kMergeElems && kMergeElems % d == 0 &&
      kMergeElems / d <= kMergeMaxRows) {
    const int rpb = kMergeElems / d;
    const int iblocks = (l + rpb - 1) / rpb;
    const long long nblocks = (long long)n * h * iblocks;
    dim3 grid(capped_grid(nblocks)), block(kMergeThreads);
    const bool walk = nblocks > (long long)grid.x;
    if (blk_bf16) {
      if (walk)
        hipLaunchKernelGGL((merge_vec_kernel<true, true>), grid, block, 0, stream, out_acc,
                           lse_acc, out_blk, lse_blk, l, h, d, iblocks, nblocks);
      else
        hipLaunchKernelGGL((merge_vec_kernel<true, false>), grid, block, 0, stream, out_acc,
                           lse_acc, out_blk, lse_blk, l, h, d, iblocks, nblocks);
    } else if (walk) {
      hipLaunchKernelGGL((merge_vec_kernel<false, true>), grid, block, 0, stream, out_acc,
                         lse_acc, out_blk, lse_blk, l, h, d, iblocks, nblocks);
    } else {
      hipLaunchKernelGGL((merge_vec_kernel<false, false>), grid, block, 0, stream, out_acc,
                         lse_acc, out_blk, lse_blk, l, h, d, iblocks, nblocks);
    }
    return hipGetLastError();
  }
  int rpb = 1024 / d;
  if (rpb < 1) rpb = 1;
  if (rpb > kMergeMaxRows) rpb = kMergeMaxRows;
  const long long blocks = (rows + rpb - 1) / rpb;
  dim3 grid(capped_grid(blocks)), block(kMergeThreads);
  if (blk_bf16)
    hipLaunchKernelGGL((merge_kernel<true>), grid, block, 0, stream, out_acc,
                       lse_acc, out_blk, lse_blk, l, h, d, rows, rpb, blocks);
  else
    hipLaunchKernelGGL((merge_kernel<false>), grid, block, 0, stream, out_acc,
                       lse_acc, out_blk, lse_blk, l, h, d, rows, rpb, blocks);
  return hipGetLastError();
}

hipError_t launch_hbm_copy(const void* src, void* dst, long long n4, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_copy_kernel, dim3(capped_grid((n4 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const f32x4_t*>(src), static_cast<f32x4_t*>(dst), n4);
  return hipGetLastError();
}

hipError_t launch_acc_clear_empty(float* out_acc, const float* lse_acc, int n, int l,
                                  int h, int d, hipStream_t stream) {
  const long long rows = (long long)n * l * h;
  hipLaunchKernelGGL(acc_clear_empty_kernel, dim3(capped_grid((rows + 255) / 256)), dim3(256),
                     0, stream, out_acc, lse_acc, l, h, d, rows);
  return hipGetLastError();
}

hipError_t launch_acc_init(float* out_acc, float* lse_acc, int n, int l, int h,
                           int d, hipStream_t stream) {
  const long long n_acc = (long long)n * l * h * d;
  const long long n_lse = lse_acc != nullptr ? (long long)n * l * h : 0;
  const long long n4 = (reinterpret_cast<uintptr_t>(out_acc) % 16 == 0) ? n_acc / 4 : 0;
  hipLaunchKernelGGL(acc_init_kernel, dim3(grid_for(n_acc / 4 + 1, 256)), dim3(256),
                     0, stream, out_acc, lse_acc, n_acc, n4, n_lse);
  return hipGetLastError();
}

hipError_t launch_acc_cast(const float* out_acc, void* out, int n, int l,
                           int h, int d, bool bf16, hipStream_t stream) {
  const long long n_elem = (long long)n * l * h * d;
  dim3 grid(grid_for(n_elem / 4 + 1, 256 * 2)), block(256);
  if (bf16)
    hipLaunchKernelGGL((acc_cast_kernel<true>), grid, block, 0, stream, out_acc,
                       out, n_elem);
  else
    hipLaunchKernelGGL((acc_cast_kernel<false>), grid, block, 0, stream, out_acc,
                       out, n_elem);
  return hipGetLastError();
}

}  // namespace bea
