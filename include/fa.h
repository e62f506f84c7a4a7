/* Fused attention forward for AMD Instinct MI355X (gfx950): C ABI.
 *
 *   out = softmax(scale * Q K^T + mask) V,   lse = log sum exp(scale * Q K^T + mask)
 *
 * The operation is the forward of FlashAttention-style attention as the
 * "flashrt/fa4-cute-runtime" card describes it: section "Functions" (the
 * forward returns the output together with the per-row log-sum-exp; an
 * allocation-free entry point writes into caller-owned output for graph
 * capture), the padded fixed-shape example (a device-resident int32
 * seqused_k and grouped-query head packing), and the closing section on the
 * (batch, sequence, heads, head_dim) layout and the qualified D72 MHA and
 * D256 8-Q/1-KV-head profiles.  Masked keys contribute exactly zero
 * probability, as in the seqused attention passage of
 * "pi05_thor_decoder_fp4_e2e.md", section "Fused GeGLU FFN in the Decoder".
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named q, k, v, out, lse, seqused_k, dev_ptr is a
 *     DEVICE pointer.  The library never dereferences one on the host, never
 *     allocates, never synchronises, and never copies between host and
 *     device, so fa_fwd can be captured into a HIP graph.
 *   - All memory is owned by the caller.
 *   - Errors are returned as FA_* codes before any device work is queued;
 *     nothing is launched when a check fails.  Faults inside a kernel
 *     surface at the caller's next synchronisation, as with any HIP launch.
 *   - There is no fallback: an unsupported input is an error, never routed
 *     to another implementation.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 5

/* Status codes. */
enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* a size is < 1, Hq % Hkv != 0, or a size overflows 32-bit indexing
                             (element counts of q and k, or Sk*Hkv*D*2 bytes per batch entry, >= 2^31);
                             fa_fwd_strided: also bad strides (see there) */
  FA_ERR_UNSUPPORTED = 3, /* D not in {64, 72, 256}; variant not compiled; unknown element type */
  FA_ERR_ALIGN = 4,       /* q, k, v, out not 16-byte aligned (or strides not multiples of 8 elements);
                             lse or seqused_k not 4-byte aligned */
  FA_ERR_SCALE = 5,       /* scale not finite or not > 0 */
  FA_ERR_WORKSPACE = 6,   /* the split-KV path needs a workspace that is missing or too small */
  FA_ERR_LAUNCH = 7,      /* the HIP runtime rejected a kernel launch */
  FA_ERR_ALIAS = 8,       /* out or lse overlaps q, k, v, seqused_k or cu_seqlens_q/k, or lse
                             overlaps out (outputs are written while other workgroups still
                             read the inputs) */
  FA_ERR_SCRATCH = 9      /* fa_fwd_static: the shape's split-KV partials exceed the static
                             scratch (FA_STATIC_SCRATCH_BYTES) */
};

/* fa_fwd: one attention forward pass.
 *
 *   q          [B, Sq, Hq, D]  bf16, contiguous (head_dim fastest)
 *   k, v       [B, Sk, Hkv, D] bf16, contiguous
 *   out        [B, Sq, Hq, D]  bf16, written (round to nearest even)
 *   lse        [B, Hq, Sq]     fp32, written (natural log, scale included),
 *                              or NULL to skip it
 *   seqused_k  NULL (all Sk keys valid) or int32[B] on the device: keys
 *              j >= seqused_k[b] of batch b are neither read nor attended.
 *              Values are clamped to [0, Sk] on the device.  A row with no
 *              attended key gets out = 0 and lse = -inf.
 *   causal     0 or 1.  With 1, query i attends key j only when
 *              j <= i + (n_b - Sq), n_b the valid keys of batch entry b
 *              (Sk, or seqused_k[b]): the last query row lines up with the
 *              last valid key, so Sq == Sk without seqused_k is the usual
 *              j <= i prefill mask (the causal prefill of "Model Demo: PI0.5
 *              End-to-End VLA Inference", section "Model stages"), and fewer
 *              queries than keys is a chunk of new positions attending a
 *              cache (decode: Sq = 1 attends every valid key).  Rows with
 *              i + n_b - Sq < 0 attend nothing (out = 0, lse = -inf).
 *   scale      softmax temperature applied to q.k (finite, > 0), passed as
 *              float; use 1/sqrt(D) for the usual scaling.
 *   Hq % Hkv == 0; query head h reads K/V head h / (Hq / Hkv).
 *   D is 64, 72 or 256.
 *   stream     HIP stream for the launch (NULL = default stream).
 *
 * Shapes with few packed query rows per compute unit take a split-KV path
 * (several workgroups per row block write partial results that a second
 * kernel on the same stream merges in fixed order) that needs a workspace
 * registered with fa_set_workspace() on the current device; fa_fwd_workspace_bytes() says how many bytes (0 when the
 * single-pass path is used).  Calls that share one workspace must not run
 * concurrently (one stream at a time per device).
 *
 * Returns FA_OK after queueing the work, or an FA_ERR_* code (nothing queued).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
           const int32_t* seqused_k, float scale, hipStream_t stream);

/* fa_fwd_static: fa_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, checks, plan, kernels and results are those of
 * fa_fwd (bit for bit); the only difference is where the split-KV path keeps
 * its partial results: in a device array inside this library, one per GPU,
 * of FA_STATIC_SCRATCH_BYTES, instead of a workspace registered with
 * fa_set_workspace.  It calls no allocator: the array exists from the
 * library's load on each GPU until the process ends, and its address is
 * looked up once per device on the first call there.
 *   - A shape whose partials need more than FA_STATIC_SCRATCH_BYTES
 *     (fa_fwd_workspace_bytes() tells) returns FA_ERR_SCRATCH, with nothing
 *     queued; use fa_fwd with a registered workspace for it.  Shapes that
 *     take the single-pass path use no scratch at all.
 *   - Every call on one GPU shares that GPU's array: calls whose execution
 *     overlaps in time on one GPU (different streams, or graph replays run
 *     concurrently) race and may return wrong results.  Serialise them (one
 *     stream).  Nothing in the array needs clearing between calls.
 * Returns FA_OK after queueing the work, or an FA_ERR_* code (FA_ERR_LAUNCH
 * also when the array's address cannot be obtained). */
#define FA_STATIC_SCRATCH_BYTES (8u << 20)
int fa_fwd_static(const void* q, const void* k, const void* v, void* out, float* lse,
                  int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
                  const int32_t* seqused_k, float scale, hipStream_t stream);

/* Element types of q, k, v and out (fa_fwd_strided). */
enum {
  FA_BF16 = 0,  /* bfloat16; out rounded to nearest even */
  FA_FP16 = 1   /* IEEE half; out rounded to nearest even */
};

/* fa_fwd_strided: fa_fwd over strided views and either element type.
 *
 * The self-attention of the GROOT action head reads the fused QKV GEMM
 * output in place (token stride 3*H*D), dropping the split copies
 * ("GROOT N1.7 update: Thor NVFP4 + FA4 performance tier", section "What is
 * in the tier"); fp16 is the other element type of the pages' attention
 * kernels (the fp16 decoder attention of "pi05_thor_decoder_fp4_e2e.md",
 * section "Fused GeGLU FFN in the Decoder"; the fp16 and bf16 FlashAttention-2
 * forwards of "deployment_rtx4090.md").
 *
 *   q, out     (batch, position, head, head_dim) views: element (b, s, h, d)
 *              at base + b*x_sb + s*x_ss + h*x_sh + d (strides in ELEMENTS;
 *              head_dim is contiguous)
 *   k, v       (batch, key, kv head, head_dim) views, same rule with their
 *              own strides
 *   dtype      FA_BF16 or FA_FP16, for q, k, v and out alike (fp32
 *              accumulation, P rounded to the element type)
 *   Everything else (lse [B, Hq, Sq] fp32 contiguous, seqused_k, causal,
 *   scale, stream, workspace) is as for fa_fwd, and the kernel variant is
 *   the one fa_fwd_plan reports.  With contiguous strides
 *   (S*H*D, H*D, D) and FA_BF16 it computes exactly what fa_fwd does.
 * Extra requirements: strides >= 0 and multiples of 8 elements (16-byte
 * rows, FA_ERR_ALIGN otherwise); sequence and head strides below 2^31
 * elements (FA_ERR_SHAPE); key rows of one head do not overlap
 * (k_ss, v_ss >= D when Sk > 1) and no two output rows overlap
 * (FA_ERR_SHAPE); Sk*k_ss*2 and Sk*v_ss*2 bytes, and the bytes from a
 * batch entry's first query row to its last, below 2^31 (FA_ERR_SHAPE);
 * out and lse must not share a byte with the span of q, k, v or seqused_k
 * (FA_ERR_ALIAS).  q, k and v may share memory (e.g. one fused QKV buffer).
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Sq, int Sk, int Hq, int Hkv, int D,
                   int64_t q_sb, int64_t q_ss, int64_t q_sh,
                   int64_t k_sb, int64_t k_ss, int64_t k_sh,
                   int64_t v_sb, int64_t v_ss, int64_t v_sh,
                   int64_t o_sb, int64_t o_ss, int64_t o_sh,
                   int dtype, int causal, const int32_t* seqused_k, float scale, hipStream_t stream);

/* fa_fwd_varlen: attention over a packed batch of variable-length
 * sequences, the varlen forward listed beside the fixed-shape one in the
 * "flashrt/fa4-cute-runtime" card, section "Functions" (multi-view or
 * multi-request packing without padding).
 *
 *   q, out        [total_q, Hq, D] contiguous, the B sequences' queries back
 *                 to back; out rows that belong to no sequence are not written
 *   k, v          [total_k, Hkv, D] contiguous, the sequences' keys
 *   lse           [Hq, total_q] fp32 (natural log, scale included), or NULL
 *   cu_seqlens_q, cu_seqlens_k
 *                 int32[B + 1] on the DEVICE: sequence b has the query rows
 *                 [cu_q[b], cu_q[b+1]) and the keys [cu_k[b], cu_k[b+1]).
 *                 Meant to be non-decreasing from 0; the kernels clamp every
 *                 span into its tensor (start to [0, total], end to
 *                 [start, total]) and cut it at max_seqlen, so no value can
 *                 address memory outside the tensors (spans that overlap
 *                 because the offsets run backwards give unspecified rows).
 *   max_seqlen_q, max_seqlen_k
 *                 host bounds on the span lengths; the grid is planned for
 *                 them (and the kernel variant is fa_fwd_plan's for
 *                 B, max_seqlen_q, max_seqlen_k)
 *   dtype         FA_BF16 or FA_FP16
 *   causal        as for fa_fwd within each sequence: query i of a sequence
 *                 with n keys attends keys j <= i + (n - its query count)
 *   A sequence without keys gives out = 0 and lse = -inf on its rows.
 * Workspace: fa_fwd_workspace_bytes(B, max_seqlen_q, max_seqlen_k, Hq, Hkv,
 * D, causal).  Checks and codes as for fa_fwd (sizes: total_q*Hq*D and
 * total_k*Hkv*D elements and max_seqlen_k*Hkv*D*2 bytes below 2^31;
 * cu_seqlens 4-byte aligned; out/lse must not overlap q, k, v or the
 * cu_seqlens arrays). */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int B, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int Hq, int Hkv, int D, int dtype, int causal, float scale, hipStream_t stream);

/* Bytes of workspace fa_fwd needs for this shape (0: none).  Pure host
 * arithmetic; returns 0 for invalid shapes as well.  The same figure holds
 * for fa_fwd_strided (the workspace does not depend on strides or dtype). */
size_t fa_fwd_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal);

/* Registers a caller-owned device buffer as the split-KV workspace of the
 * current HIP device (replacing any earlier one; NULL/0 unregisters).  The
 * buffer must be 256-byte aligned; it needs no initialisation.  It must
 * outlive every fa_fwd call queued with it, and calls sharing it must not
 * overlap in time (e.g. run them on one stream).  Not thread-safe against
 * concurrent fa_fwd calls.
 * Returns FA_OK, FA_ERR_NULL for a NULL pointer with bytes > 0, or
 * FA_ERR_LAUNCH when no HIP device is current. */
int fa_set_workspace(void* dev_ptr, size_t bytes);

/* fa_fwd_nvfp4: fa_fwd with the output quantised to NVFP4 for the output
 * projection, in the same launch ("pi05_thor_decoder_fp4_e2e.md", section
 * "Implemented Path": dynamic NVFP4 quantisation of the attention output
 * before O; "GROOT N1.7 update: Thor NVFP4 + FA4 performance tier", section
 * "What is in the tier": per-16-element, no calibration; the same page as
 * the first, section "E0M3 Uniform-INT4 Decoder Weights": per-16 UE4M3
 * scales at amax over the grid maximum).
 *   out_fp4  [B, Sq, Hq, D/2] bytes, written: the E2M1 codes of each
 *            (token, head) row, element 2i in the low nibble of byte i
 *            (4-byte aligned)
 *   out_sf   [B, Sq, Hq, D/16] bytes, written: one UE4M3 scale per 16
 *            consecutive head-dim elements
 * A block's scale is amax/6 (fp32) rounded to UE4M3 (nearest, ties to the
 * even code, at most 448); its elements are x / (decoded scale) (fp32)
 * rounded to E2M1 (nearest, ties to the even code, at most 6 in magnitude;
 * sign bit when x < 0), x the fp32 attention output before any rounding;
 * a scale that rounds to zero gives zero codes.  q, k, v are bf16 and
 * contiguous; D must be 64 or 256 (a multiple of 16 with a compiled
 * variant; FA_ERR_UNSUPPORTED otherwise).  Everything else (lse,
 * seqused_k, causal, scale, stream, workspace, checks and codes) is as for
 * fa_fwd; out_fp4, out_sf and lse must not overlap each other or q, k, v,
 * seqused_k (FA_ERR_ALIAS). */
int fa_fwd_nvfp4(const void* q, const void* k, const void* v, void* out_fp4, void* out_sf, float* lse,
                 int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
                 const int32_t* seqused_k, float scale, hipStream_t stream);

/* Tuning and testing entry points.  fa_fwd picks its kernel variant from
 * the shape alone; these name one explicitly so that every compiled variant
 * can be timed and checked:
 *   qt   rows per wavefront / 16   (1 or 2)
 *   nw   wavefronts per workgroup  (2, 4 or 8)
 *   kw   1: the wavefronts own different rows and share the K/V tiles;
 *        nw: all wavefronts own the same rows and split the keys between
 *        them, each streaming its own tiles (nst 1: whole-tile buffers,
 *        2: piecewise refill, 3: piecewise refill through one ring buffer
 *        per wavefront, 80 KiB of LDS, two workgroups per compute unit);
 *        2 with nw = 4 or 8: two groups of nw/2 wavefronts on the same
 *        rows, each group sharing its own K/V tiles and taking every other
 *        key tile, merged at the end (nst 2)
 *   bn   keys per tile             (32, 64 or 128)
 *   nst  K/V tile stages in LDS    (1, 2, 3 or 4)
 *   kps  keys per split-KV range   (0: single pass; else a multiple of bn)
 * A combination that is not compiled returns FA_ERR_UNSUPPORTED.  Other
 * arguments, checks and errors are those of fa_fwd. */
int fa_fwd_variant(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
                   const int32_t* seqused_k, float scale, int qt, int nw, int kw, int bn, int nst,
                   int kps, hipStream_t stream);

/* Workspace bytes for fa_fwd_variant with that variant (0: none or invalid). */
size_t fa_fwd_variant_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
                                      int qt, int nw, int kw, int bn, int nst, int kps);

/* The variant fa_fwd chooses for a shape, written to *qt, *nw, *kw, *bn,
 * *nst, *kps.  Returns FA_OK or the shape error fa_fwd would return. */
int fa_fwd_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
                int* qt, int* nw, int* kw, int* bn, int* nst, int* kps);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_string(int code);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
