/*
 * attn.h - C ABI of the MI355X (gfx950) blockwise exact-attention library.
 *
 * Exact scaled-dot-product attention computed blockwise with an online
 * softmax, returning both the output O and the natural-log log-sum-exp LSE of
 * every query row; the (O, LSE) merge of partial results; the accumulator
 * set-up and final cast of one device's ring-attention share; and the
 * backward pass.
 *
 * Sources (page title, then the function on the page):
 *   - "flash_sharding.py" (flash_attn_jax): partition_fwd / partition_bwd
 *     (the kernel interface fwd(q,k,v; softmax_scale, is_causal,
 *     window_size) -> (o, lse) and bwd(do,q,k,v,o,lse; ...) -> (dq,dk,dv);
 *     O sharded like q, LSE laid out [n,h,l]); ring_fwd (accumulator start
 *     O = 0, LSE = -inf; skipped chunk = (0, -inf); log1p merge; final cast
 *     of O to the query dtype); ring_bwd (gradients cast to the query dtype).
 *   - "picotron/parallel/context_parallel.py": ring_attention_forward and
 *     ring_attention_backward (the math), update_out_and_lse (merge; block
 *     output upcast to fp32), RingAttention._repeat_kv (grouped-query heads).
 *
 * Conventions shared by every call
 *   - Every tensor pointer is device memory owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no pointer after the call
 *     returns.  All tensors are dense and row-major (contiguous).
 *   - Layouts: q, out, dout, dq        [n, l_q, h,    d]
 *              k, v, dk, dv            [n, l_k, h_kv, d]
 *              lse                     [n, h, l_q]   float32
 *              out_acc                 [n, l, h, d]  float32
 *   - dtype selects the element type of q, k, v, out, dout, dq, dk, dv:
 *     ATTN_BF16 (bfloat16) or ATTN_F32 (float32).  LSE and the merge
 *     accumulator are always float32.  Outputs are rounded to nearest even.
 *   - Grouped-query heads: h must be a multiple of h_kv and query head hq
 *     reads key/value head hq / (h / h_kv) (consecutive query heads share a
 *     key/value head).  h_kv == 1 is multi-query attention.
 *   - Masking uses absolute positions qpos = q_offset + i for query row i and
 *     kpos = k_offset + j for key row j.  Key j is allowed for row i when
 *       (causal == 0 || kpos <= qpos) &&
 *       (win_l < 0 || kpos >= qpos - win_l) &&
 *       (win_r < 0 || kpos <= qpos + win_r).
 *     Window bounds are inclusive; a negative side is unbounded, so
 *     (win_l, win_r) = (-1, -1) means no window.  Only q_offset - k_offset
 *     matters.  Offsets 0 give top-left causal alignment.
 *   - A query row with no allowed key gets O = 0 and LSE = -inf, and zero
 *     gradients.
 *   - Empty inputs: n, l_q, l_k (and l of the accumulator calls) may be 0;
 *     h, h_kv and d may not.  A pointer may be NULL exactly when its tensor
 *     has no elements.  With no query rows a call writes nothing; with no
 *     keys (l_k = 0) every row is empty: attn_fwd writes O = 0 and
 *     LSE = -inf, attn_fwd_acc merges the empty block like attn_merge does
 *     (rows with a result keep it, rows at LSE -inf get O = 0), attn_bwd
 *     writes dQ = 0 (and dK = dV = 0 when
 *     l_q = 0 instead), attn_bwd_acc adds nothing.  These are the pages'
 *     fully-masked conventions applied to a chunk with no rows or no keys.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it and returns without synchronising.  The
 *     library keeps no global state: calls on different streams from
 *     different host threads are independent.
 *   - Every argument is checked before any HIP call; on error nothing is
 *     launched and a nonzero status is returned.  ATTN_ERR_HIP reports a
 *     failed launch (hipGetLastError after the launch).
 */
#ifndef BLOCKWISE_EXACT_ATTENTION_AMD_ATTN_H
#define BLOCKWISE_EXACT_ATTENTION_AMD_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a pointer to a non-empty tensor is NULL           */
  ATTN_ERR_SHAPE = 2,       /* a size is negative, h, h_kv or d is 0,
                               h % h_kv != 0, sizes overflow, a row of q
                               (h * d) exceeds 32 MiB in float32, a launch
                               would exceed 2^31 workgroups or 2^32 work-items
                               (n*l_q*h >= 2^30 query rows or n*l_k*h_kv >= 2^30
                               key rows), or a chunk count outside
                               1..ATTN_RING_MAX_CHUNKS                           */
  ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, unknown dtype or non-finite
                               scale                                             */
  ATTN_ERR_HIP = 4,         /* the HIP runtime reported a launch failure         */
  ATTN_ERR_WORKSPACE = 5,   /* workspace smaller than required (or NULL when
                               required)                                         */
  ATTN_ERR_ALIAS = 6,       /* an input buffer overlaps an output buffer         */
  ATTN_ERR_ALIGN = 7        /* a tensor pointer is not 16-byte aligned (LSE
                               pointers: 4-byte aligned)                          */
};

enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1 };

/*
 * attn_fwd - exact attention forward, blockwise with an online softmax.
 * (flash_sharding.py: the fwd kernel called by partition_fwd and ring_fwd;
 *  picotron: ring_attention_forward.)
 *
 *   O[b,i,hq,:] = sum_j P_ij v[b,j,g,:],  P_ij = exp(s_ij - LSE[b,hq,i]),
 *   s_ij = scale * <q[b,i,hq,:], k[b,j,g,:]>,  LSE = log sum_{allowed j} exp(s_ij),
 *   g = hq / (h / h_kv), sums over allowed keys only.
 *
 *   q   [n,l_q,h,d]     in   dtype
 *   k,v [n,l_k,h_kv,d]  in   dtype
 *   out [n,l_q,h,d]     out  dtype (rounded to nearest even)
 *   lse [n,h,l_q]       out  float32, natural log, -inf for empty rows
 *   d in {64, 128}; any finite scale (the pages use 1/sqrt(d)).
 * out and lse must not overlap q, k or v.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int n, int l_q, int l_k, int h, int h_kv, int d,
             float scale, int causal, int win_l, int win_r,
             long long q_offset, long long k_offset, void* stream, int dtype);

/*
 * attn_merge - merge a partial result over one key chunk into an accumulator
 * over other keys (flash_sharding.py ring_fwd, log1p form; picotron
 * update_out_and_lse, sigmoid form - the two are equal):
 *   lse = max(a,b) + log1p(exp(min(a,b) - max(a,b)))
 *   out_acc = out_acc * exp(a - lse) + float(out_blk) * exp(b - lse)
 * with a = lse_acc, b = lse_blk per row (b, hq, i).  If b = -inf and a is
 * finite the row is left unchanged; if a = -inf and b is finite the row
 * becomes (out_blk, b); if both are -inf the row becomes the empty result
 * (O = 0, LSE = -inf).  A row at a = -inf is written without reading
 * out_acc, so an accumulator whose O holds anything (NaN included) is safe
 * wherever its LSE is -inf.
 *
 *   out_acc [n,l,h,d] float32  in/out      lse_acc [n,h,l] float32 in/out
 *   out_blk [n,l,h,d] blk_dtype in         lse_blk [n,h,l] float32 in
 *   any d >= 1.  out_blk / lse_blk must not overlap out_acc / lse_acc.
 */
int attn_merge(float* out_acc, float* lse_acc, const void* out_blk,
               const float* lse_blk, int n, int l, int h, int d, int blk_dtype,
               void* stream);

/*
 * attn_fwd_acc - one ring step fused: attention of q against this key/value
 * chunk, merged straight into the ring accumulator (flash_sharding.py
 * ring_fwd and picotron ring_attention_forward: the fwd call on the chunk
 * followed by the merge).  The result equals attn_fwd into a block (O, LSE)
 * followed by attn_merge of that block, except that the block's O is merged
 * in float32 instead of being rounded to the query dtype first; the same
 * -inf guards apply (a row with no allowed key in this chunk is left alone,
 * or set to O = 0 when the accumulator row is at -inf too; an accumulator
 * row at -inf is replaced, whatever it held).
 *
 *   q       [n,l_q,h,d]     in      dtype (ATTN_BF16 or ATTN_F32)
 *   k,v     [n,l_k,h_kv,d]  in      dtype
 *   out_acc [n,l_q,h,d]     in/out  float32
 *   lse_acc [n,h,l_q]       in/out  float32, natural log
 *   d in {64, 128}; any finite scale; masking as for attn_fwd.
 * out_acc and lse_acc must not overlap each other or q, k, v.  Rows of
 * different query tiles are merged by different workgroups, so two calls on
 * the same accumulator must be ordered (one stream, or an event between).
 */
int attn_fwd_acc(const void* q, const void* k, const void* v, float* out_acc,
                 float* lse_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                 float scale, int causal, int win_l, int win_r,
                 long long q_offset, long long k_offset, void* stream, int dtype);

/*
 * attn_fwd_kernel_name - which kernel attn_fwd (fused = 0) or attn_fwd_acc
 * (fused = 1) launches for these arguments: the template instantiation as
 * kernel traces name it (a static string), or NULL when the call would be
 * rejected or would launch no attention kernel (no rows or no keys).  For
 * profiling and reports; launches nothing.
 */
const char* attn_fwd_kernel_name(int n, int l_q, int l_k, int h, int h_kv, int d,
                                 float scale, int causal, int win_l, int win_r,
                                 long long q_offset, long long k_offset, int dtype,
                                 int fused);

/*
 * attn_fwd_ring - one device's whole ring-attention share in one launch
 * (flash_sharding.py ring_fwd: the loop over the key/value chunks that pass
 * around the ring, each attended with its own absolute offset and merged
 * into the running (O, LSE); picotron RingAttentionFunc.forward).  The
 * online softmax runs across the chunks in the order given, so no
 * accumulator leaves the registers: the result is attn_fwd over the keys of
 * all chunks together, key j of chunk c at absolute position
 * k_offsets[c] + j (what attn_acc_init, attn_fwd_acc per chunk and
 * attn_acc_cast give, up to rounding order).
 *
 *   q            [n,l_q,h,d]     in   dtype
 *   k_chunks[c], v_chunks[c]
 *                [n,l_k_chunks[c],h_kv,d]  in  dtype, device pointers
 *   k_chunks, v_chunks, l_k_chunks, k_offsets: host arrays of n_chunks
 *                entries, read during the call only
 *   out          [n,l_q,h,d]     out  dtype
 *   lse          [n,h,l_q]       out  float32, natural log, -inf for rows
 *                with no allowed key in any chunk (O = 0 there)
 *   1 <= n_chunks <= ATTN_RING_MAX_CHUNKS (else ATTN_ERR_SHAPE); a chunk may
 *   have l_k_chunks[c] = 0 (it adds nothing); d in {64, 128}; masking as for
 *   attn_fwd with q_offset and each chunk's k_offsets[c].
 * out and lse must not overlap q or any chunk.  Each chunk is checked as
 * attn_fwd checks k and v.  ATTN_F32: out and lse themselves serve as the
 * float32 accumulator, set to the empty result and then merged into by one
 * fused step (as attn_fwd_acc) per chunk with keys, in the order given:
 * 1 + (chunks with keys) launches instead of one.
 */
#define ATTN_RING_MAX_CHUNKS 16
int attn_fwd_ring(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                  const int* l_k_chunks, const long long* k_offsets, int n_chunks,
                  void* out, float* lse, int n, int l_q, int h, int h_kv, int d,
                  float scale, int causal, int win_l, int win_r, long long q_offset,
                  void* stream, int dtype);

/*
 * attn_hbm_copy - a plain device copy of `bytes` bytes (a multiple of 16)
 * by 16-byte nontemporal loads and stores: what a streaming elementwise
 * kernel reaches on this GPU, the bandwidth reference the merge is measured
 * against.  Not part of the attention path.  src and dst must not overlap.
 */
int attn_hbm_copy(const void* src, void* dst, long long bytes, void* stream);

/*
 * attn_acc_init - set a ring accumulator to the empty result, O = 0 and
 * LSE = -inf (flash_sharding.py ring_fwd, its initial o and lse).
 *   out_acc [n,l,h,d] float32 out; lse_acc [n,h,l] float32 out, or NULL to
 *   zero out_acc only (the gradient accumulators of attn_bwd_acc).
 */
int attn_acc_init(float* out_acc, float* lse_acc, int n, int l, int h, int d,
                  void* stream);

/*
 * attn_acc_cast - final cast of the ring accumulator to the query dtype,
 * rounding to nearest even (flash_sharding.py ring_fwd, o.astype(q.dtype)).
 *   out_acc [n,l,h,d] float32 in; out [n,l,h,d] dtype out (may not overlap).
 */
int attn_acc_cast(const float* out_acc, void* out, int n, int l, int h, int d,
                  int dtype, void* stream);

/*
 * attn_bwd - exact attention backward by recomputation from the saved LSE
 * (picotron ring_attention_backward; flash_sharding.py bwd argument order
 * dout, q, k, v, out, lse and gradients in the query dtype):
 *   P = exp(S - LSE), D_i = sum_c dout_ic out_ic, dP = dout V^T,
 *   dS = P * (dP - D) (0 where masked), dQ = scale dS K, dK = scale dS^T Q,
 *   dV = P^T dout; with grouped heads dK and dV of a key/value head sum over
 *   the query heads that read it.  Accumulation is float32.
 *
 *   dtype ATTN_BF16 (MFMA kernels) or ATTN_F32 (float32 FMA kernels, every
 *   product and sum in float32).
 *   dout, q, out [n,l_q,h,d] dtype in;  k, v [n,l_k,h_kv,d] dtype in
 *   lse [n,h,l_q] float32 in (as written by attn_fwd)
 *   dq [n,l_q,h,d], dk, dv [n,l_k,h_kv,d] dtype out
 *   workspace: device scratch of at least attn_bwd_workspace_bytes(...) bytes,
 *   owned by the caller; its contents on entry do not matter.
 * Outputs must not overlap inputs, the workspace or each other.
 */
int attn_bwd(const void* dout, const void* q, const void* k, const void* v,
             const void* out, const float* lse, void* dq, void* dk, void* dv,
             int n, int l_q, int l_k, int h, int h_kv, int d,
             float scale, int causal, int win_l, int win_r,
             long long q_offset, long long k_offset,
             void* workspace, size_t workspace_bytes, void* stream, int dtype);

/*
 * attn_bwd_acc - one step of the ring backward as one device sees it
 * (picotron ring_attention_backward; flash_sharding.py ring_bwd): the
 * gradient contributions of this key/value chunk, added to float32
 * accumulators instead of written:
 *   dq_acc += scale dS K,  dk_acc += scale dS^T Q,  dv_acc += P^T dout,
 * with P = exp(S - lse), D = rowsum(dout * out), dS = P (dP - D), as in
 * attn_bwd.  For a ring step, out and lse are the query rows' results over
 * the whole sequence (the forward ring share's final O and LSE), so that P is
 * the global softmax restricted to this chunk; summing the steps then gives
 * the full gradients.  dk_acc / dv_acc of a chunk collect the contributions
 * of every query block that reads it (in a real ring they travel with the
 * chunk).
 *   dout, q, out [n,l_q,h,d] dtype; k, v [n,l_k,h_kv,d] dtype; lse [n,h,l_q]
 *   dq_acc [n,l_q,h,d] float32 in/out; dk_acc, dv_acc [n,l_k,h_kv,d]
 *   float32 in/out; workspace as for attn_bwd; dtype ATTN_BF16 or ATTN_F32.
 * The accumulators must not overlap the inputs, the workspace or each other;
 * calls that add to the same accumulator must be ordered on one stream.
 */
int attn_bwd_acc(const void* dout, const void* q, const void* k, const void* v,
                 const void* out, const float* lse, float* dq_acc, float* dk_acc,
                 float* dv_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                 float scale, int causal, int win_l, int win_r,
                 long long q_offset, long long k_offset,
                 void* workspace, size_t workspace_bytes, void* stream, int dtype);

/* Bytes of workspace attn_bwd / attn_bwd_acc need for these sizes (0 on
 * invalid sizes, and 0 when n, l_q or l_k is 0: then no kernel reads it and
 * workspace may be NULL): D and LSE per query row and, when the key tiles alone would
 * give the dK/dV kernel fewer than 512 workgroups, per-split float32 dK/dV
 * partials (summed in a fixed order, so results stay bitwise repeatable). */
size_t attn_bwd_workspace_bytes(int n, int l_q, int l_k, int h, int h_kv, int d);

/*
 * attn_bwd_prepare + attn_bwd_acc_prepared - the ring backward share with
 * its per-row preprocessing done once (picotron ring_attention_backward
 * forms D = rowsum(dO * O) from the saved global output once, before the
 * loop over the chunks; flash_sharding.py ring_bwd likewise passes the same
 * (o, lse, do) to every chunk's backward).
 *
 * attn_bwd_prepare writes, for the query rows of (dout, out, lse), D and the
 * LSE in base-2 units into the first attn_bwd_prepare_bytes(n, l_q, h)
 * bytes of `workspace` (at least that many; 16-byte aligned).  Shapes as
 * for attn_bwd; dtype ATTN_BF16 or ATTN_F32 (the rows are the same float32
 * values either way, so a share prepares with the dtype of its dout, out).
 *
 * attn_bwd_acc_prepared is attn_bwd_acc (same arguments and workspace
 * size) without that preprocessing: it reads D and the LSE from the
 * workspace, which must hold what attn_bwd_prepare wrote for the same
 * dout, out, lse and sizes, untouched since (the calls in between may be
 * other attn_bwd_acc_prepared calls of the share, which only write the
 * rest of the workspace).  Results equal attn_bwd_acc's bit for bit.
 */
size_t attn_bwd_prepare_bytes(int n, int l_q, int h);
int attn_bwd_prepare(const void* dout, const void* out, const float* lse, int n, int l_q,
                     int h, int d, void* workspace, size_t workspace_bytes, void* stream,
                     int dtype);
int attn_bwd_acc_prepared(const void* dout, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, float* dq_acc, float* dk_acc,
                          float* dv_acc, int n, int l_q, int l_k, int h, int h_kv, int d,
                          float scale, int causal, int win_l, int win_r, long long q_offset,
                          long long k_offset, void* workspace, size_t workspace_bytes,
                          void* stream, int dtype);

/*
 * attn_bwd_ring - one device's whole ring backward share in three launches
 * (picotron RingAttentionFunc.backward / ring_attention_backward: the
 * gradient of the share's queries against every chunk, D formed once from
 * the saved global output; flash_sharding.py ring_bwd: dq summed over the
 * chunks and cast to the query dtype).  For the share's query rows q with
 * the forward share's final (out, lse) and the incoming dout:
 *   dq            [n,l_q,h,d]    out  dtype: scale * sum over all chunks of
 *                                     dS K (written, not accumulated)
 *   dk_acc_chunks[c], dv_acc_chunks[c]
 *                 [n,l_k_chunks[c],h_kv,d]  in/out  float32: chunk c's dK and
 *                                     dV from these queries are ADDED (in a
 *                                     ring these accumulators travel with the
 *                                     chunk)
 *   k_chunks, v_chunks, l_k_chunks, k_offsets as for attn_fwd_ring; the
 *   pointer arrays (host, read during the call) hold n_chunks entries,
 *   1 <= n_chunks <= ATTN_RING_MAX_CHUNKS.
 *   workspace: at least attn_bwd_prepare_bytes(n, l_q, h) bytes of device
 *   scratch (contents on entry do not matter).
 * Equal, up to rounding order, to attn_bwd_acc per chunk with dQ accumulated
 * in float32 and cast at the end.  dout, q, out, the chunks and dq all in
 * dtype; d in {64, 128}.  ATTN_F32: dq itself is the float32 accumulator
 * (cleared, then D and the base-2 LSE prepared once and one accumulating
 * backward run per chunk with keys: 2 + 2 x (chunks with keys) launches).
 * No output may overlap an input or another output.
 */
int attn_bwd_ring(const void* dout, const void* q, const void* out, const float* lse,
                  const void* const* k_chunks, const void* const* v_chunks,
                  const int* l_k_chunks, const long long* k_offsets,
                  float* const* dk_acc_chunks, float* const* dv_acc_chunks, int n_chunks,
                  void* dq, int n, int l_q, int h, int h_kv, int d, float scale, int causal,
                  int win_l, int win_r, long long q_offset, void* workspace,
                  size_t workspace_bytes, void* stream, int dtype);

/*
 * attn_bwd_static - attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the workspace taken
 * from a static array of ATTN_BWD_STATIC_MAX_WORKSPACE bytes that the
 * library holds on each device it runs on until the process ends.  The
 * call allocates and frees nothing.
 *
 *   Arguments as for attn_bwd, without workspace and workspace_bytes.
 *   Returns ATTN_ERR_WORKSPACE when attn_bwd_workspace_bytes(...) for these
 *   sizes exceeds ATTN_BWD_STATIC_MAX_WORKSPACE (nothing is launched), and
 *   ATTN_ERR_HIP when the device of `stream` cannot be queried.
 * Every call on one device shares that device's array: calls that overlap
 * in time on one device (different streams without ordering between them,
 * or different host threads) race and give wrong gradients.  Order them on
 * one stream, or use attn_bwd with a workspace per stream.
 */
#define ATTN_BWD_STATIC_MAX_WORKSPACE (64 << 20)
int attn_bwd_static(const void* dout, const void* q, const void* k, const void* v,
                    const void* out, const float* lse, void* dq, void* dk, void* dv,
                    int n, int l_q, int l_k, int h, int h_kv, int d, float scale,
                    int causal, int win_l, int win_r, long long q_offset,
                    long long k_offset, void* stream, int dtype);

/* Static, human-readable name of a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKWISE_EXACT_ATTENTION_AMD_ATTN_H */
