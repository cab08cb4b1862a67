// Internal launch interface between the C ABI layer (api.hip) and the kernel
// files.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bea {

// One key/value chunk of a forward call: its tensors [n, l_k, h_kv, d]
// (bf16) and the mask bounds of its keys (allowed iff dlo <= j - i <= dhi
// and j < l_k, j counted within the chunk).
constexpr int kMaxChunks = 16;
struct FwdChunk {
  const uint16_t* k;
  const uint16_t* v;
  int l_k;
  int dlo, dhi;
};

struct AttnShape {
  int n, l_q, l_k, h, h_kv, d;
  float scale;
  int dlo, dhi;   // allowed iff dlo <= j - i <= dhi (and j < l_k)
  int causal;     // used only for the longest-first tile order
};

// acc != nullptr: merge the result into the fp32 accumulator (acc, lse_acc)
// instead of writing out and lse.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v,
                           void* out, float* lse, const AttnShape& s,
                           hipStream_t stream, float* acc = nullptr,
                           float* lse_acc = nullptr);
// The software-pipelined bf16 forward over n_chunks (1..kMaxChunks) key
// chunks visited in order by one online softmax; acc != nullptr merges the
// result into the fp32 accumulator (one chunk only).  force_ksplit 1 or 2 overrides the
// schedule choice (0: choose).
hipError_t launch_fwd_pipe(const void* q, const FwdChunk* chunks, int n_chunks, void* out,
                           float* lse, const AttnShape& s, hipStream_t stream,
                           float* acc = nullptr, float* lse_acc = nullptr,
                           int force_ksplit = 0);
// Whether the pipelined kernel is the faster one for these chunks (long key
// loops per q tile); otherwise launch_fwd_bf16 is.
bool fwd_pipe_preferred(const FwdChunk* chunks, int n_chunks, const AttnShape& s);
// Names of the kernel instantiations the launchers above would choose.
const char* fwd_bf16_kernel_name(const AttnShape& s, bool acc);
const char* fwd_pipe_kernel_name(const FwdChunk* chunks, int n_chunks, const AttnShape& s,
                                 bool acc);
// float32 forward; acc != nullptr merges into the accumulator as above.
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v,
                          void* out, float* lse, const AttnShape& s,
                          hipStream_t stream, float* acc = nullptr,
                          float* lse_acc = nullptr);

// A launch grid of min(blocks, 2^20) blocks (at least 1) for the kernels
// that walk their blocks in several passes when there are more.
unsigned capped_grid(long long blocks);

hipError_t launch_merge(float* out_acc, float* lse_acc, const void* out_blk,
                        const float* lse_blk, int n, int l, int h, int d,
                        bool blk_bf16, hipStream_t stream);
// n4 16-byte words from src to dst (the bandwidth reference of the merge).
hipError_t launch_hbm_copy(const void* src, void* dst, long long n4, hipStream_t stream);
// The merge of an all-empty block: accumulator rows whose LSE is -inf get
// O = 0, the others are left alone.
hipError_t launch_acc_clear_empty(float* out_acc, const float* lse_acc, int n, int l,
                                  int h, int d, hipStream_t stream);
hipError_t launch_acc_init(float* out_acc, float* lse_acc, int n, int l, int h,
                           int d, hipStream_t stream);
hipError_t launch_acc_cast(const float* out_acc, void* out, int n, int l,
                           int h, int d, bool bf16, hipStream_t stream);

size_t bwd_workspace_bytes(int n, int l_q, int l_k, int h, int h_kv, int d);
// Leading bytes of every backward workspace that hold the per-row D and
// LSE * log2(e).
size_t bwd_prepared_bytes(int n, int l_q, int h);
// Where those rows sit in a workspace: D at *dd, LSE * log2(e) at *lse2.
void bwd_prepared_rows(void* workspace, int n, int l_q, int h, float** dd, float** lse2);
// Writes those rows (D = rowsum(dout * out), LSE in log2 units) into the
// workspace; dout and out bf16, or float32 for the _f32 form.
hipError_t launch_bwd_prepare(const void* dout, const void* out, const float* lse, int n,
                              int l_q, int h, int d, void* workspace, hipStream_t stream);
hipError_t launch_bwd_f32_prepare(const void* dout, const void* out, const float* lse, int n,
                                  int l_q, int h, int d, void* workspace, hipStream_t stream);
// The float32 backward: dq, dk, dv written (acc: added to) in float32; the
// workspace's prepared rows are formed first unless `prepared`.
hipError_t launch_bwd_f32(const void* dout, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, float* dq, float* dk, float* dv,
                          const AttnShape& s, void* workspace, bool acc, bool prepared,
                          hipStream_t stream);
// One key/value chunk of the ring backward share: its tensors, its fp32 dK
// and dV accumulators (gradients are added), length and mask bounds.
struct BwdChunkArgs {
  const void* k;
  const void* v;
  float* dk_acc;
  float* dv_acc;
  int l_k;
  int dlo, dhi;
};
// The whole ring backward share in three launches: D and the base-2 LSE into
// the workspace (bwd_prepared_bytes), every chunk's dK/dV added to its
// accumulators, dQ over all chunks written (bf16) to dq.  Chunks non-empty,
// 1..kMaxChunks of them.
hipError_t launch_bwd_ring(const void* dout, const void* q, const void* out, const float* lse,
                           const BwdChunkArgs* chunks, int n_chunks, void* dq,
                           const AttnShape& s, void* workspace, hipStream_t stream);
// dq_acc != nullptr: add the gradients to the fp32 accumulators (dq_acc,
// dk_acc, dv_acc) instead of writing dq, dk, dv.  prepared: the workspace
// already holds the rows launch_bwd_prepare writes (not recomputed).
hipError_t launch_bwd(const void* dout, const void* q, const void* k,
                      const void* v, const void* out, const float* lse,
                      void* dq, void* dk, void* dv, const AttnShape& s,
                      void* workspace, bool bf16, hipStream_t stream,
                      float* dq_acc = nullptr, float* dk_acc = nullptr,
                      float* dv_acc = nullptr, bool prepared = false);

}  // namespace bea
