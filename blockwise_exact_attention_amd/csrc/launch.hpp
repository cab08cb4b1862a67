// Internal launch interface between the C ABI layer (api.hip) and the kernel
// files.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace bea {

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
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v,
                          void* out, float* lse, const AttnShape& s,
                          hipStream_t stream);

hipError_t launch_merge(float* out_acc, float* lse_acc, const void* out_blk,
                        const float* lse_blk, int n, int l, int h, int d,
                        bool blk_bf16, hipStream_t stream);
// The merge of an all-empty block: accumulator rows whose LSE is -inf get
// O = 0, the others are left alone.
hipError_t launch_acc_clear_empty(float* out_acc, const float* lse_acc, int n, int l,
                                  int h, int d, hipStream_t stream);
hipError_t launch_acc_init(float* out_acc, float* lse_acc, int n, int l, int h,
                           int d, hipStream_t stream);
hipError_t launch_acc_cast(const float* out_acc, void* out, int n, int l,
                           int h, int d, bool bf16, hipStream_t stream);

size_t bwd_workspace_bytes(int n, int l_q, int l_k, int h, int h_kv, int d);
// dq_acc != nullptr: add the gradients to the fp32 accumulators (dq_acc,
// dk_acc, dv_acc) instead of writing dq, dk, dv.
hipError_t launch_bwd(const void* dout, const void* q, const void* k,
                      const void* v, const void* out, const float* lse,
                      void* dq, void* dk, void* dv, const AttnShape& s,
                      void* workspace, bool bf16, hipStream_t stream,
                      float* dq_acc = nullptr, float* dk_acc = nullptr,
                      float* dv_acc = nullptr);

}  // namespace bea
