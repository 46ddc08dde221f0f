/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * The operation is exact scaled dot-product attention, defined on the
 * "FlashAttention" page (systems-analysis.ru), section "Problem of standard
 * attention":  O = softmax(scale * Q K^T) V  per batch entry b and head h,
 * with scale = 1/sqrt(d) in the usual case. The library computes it in one
 * fused, tiled kernel with a block-wise ("online") softmax (same page,
 * sections "Tiling", "Online softmax" and "Fusing into one CUDA kernel"), so
 * the N x N score matrix is never written to memory and the only extra output
 * is one logsumexp value per query row (O(N) memory, section "Complexity and
 * optimality"). The backward recomputes the probabilities from that
 * logsumexp.
 *
 * Common conventions for every entry point:
 *   Layout     q, k, v, o, dout, dq, dk, dv are contiguous row-major
 *              [B][H][N][d] arrays (element (b,h,i,c) at ((b*H+h)*N+i)*d+c);
 *              lse is a contiguous [B][H][N] float array.
 *   Memory     every pointer is a DEVICE pointer on the current HIP device.
 *              The caller allocates and owns every buffer, including the
 *              backward workspace; the library never allocates or frees
 *              memory and keeps no mutable global state, so calls are
 *              re-entrant and thread-safe.
 *   Alignment  tensor pointers must be 16-byte aligned, lse 4-byte aligned.
 *   Masking    causal != 0 keeps key j for query i only when j <= i (square,
 *              top-left aligned); causal == 0 keeps every key.
 *   Scale      any finite scale > 0 (1/sqrt(d) for the standard attention).
 *              Zero is refused: masked scores are -inf before scaling.
 *   Sizes      B, H, N >= 0; if any of them is 0 the call does nothing and
 *              returns FA_OK. N may be any positive value (no multiple of a
 *              tile size is required). d must be 64, 128 or 256 (the
 *              largest head size the "FlashAttention" page, section
 *              "FlashAttention-2 (2023)", names among FlashAttention-2's
 *              extensions); fa_fwd_f32 takes 64 and 128 only and fa_fwd_fp8
 *              128 only.
 *   Async      work is enqueued on `stream` (0 = the null stream) and the call
 *              returns; results are valid once the stream has synchronised.
 *   Errors     every argument is checked before anything is enqueued, so on
 *              an error status nothing has been launched:
 *                FA_ERR_INVALID_ARG  null pointer with non-empty sizes,
 *                                    negative size, non-finite scale or
 *                                    scale <= 0;
 *                FA_ERR_UNSUPPORTED  d not supported, misaligned pointer, or a
 *                                    size whose index arithmetic would
 *                                    overflow (grid or N beyond 2^26);
 *                FA_ERR_WORKSPACE    backward workspace too small, null or not
 *                                    256-byte aligned;
 *                FA_ERR_HIP          the HIP runtime refused the launch.
 *   Aliasing   outputs must not overlap inputs or each other.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as the HIP runtime header (a typedef may be repeated). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,
    FA_ERR_UNSUPPORTED = 2,
    FA_ERR_WORKSPACE = 3,
    FA_ERR_HIP = 4
} fa_status_t;

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_str(fa_status_t status);

/*
 * Forward, bfloat16 storage.
 *   q, k, v  (in)  bf16 [B][H][N][d].
 *   o        (out) bf16 [B][H][N][d]: O = P V with P = softmax(scale Q K^T)
 *                  (masked when causal), rounded to nearest even once.
 *   lse      (out) fp32 [B][H][N]: natural-log logsumexp of the scaled,
 *                  masked logits of each query row, ln sum_j exp(scale q_i.k_j);
 *                  the backward consumes it.
 * Q K^T runs on bf16 MFMA with fp32 accumulation; the softmax statistics,
 * probabilities and the output accumulator are fp32. The P V product takes
 * fp16 operands (more significand bits than bf16, for a sharp softmax):
 * 2^7 P and 2^-8 v, fp32 accumulation. For d = 64 and 128 the row sum that
 * normalises O and gives lse adds those fp16 probabilities in fp32, so lse
 * is within ln(1 + 2^-11) < 5e-4 of its exact value (d = 256 sums the fp32
 * probabilities for lse). So for d = 64 and 128 the values must
 * satisfy |v| < 65504 * 2^8 (about 1.68e7; larger ones overflow the fp16
 * operand and give non-finite output); at d = 256 P V takes bf16 operands
 * and any finite v is allowed.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * Forward with shared K/V heads (multi-query and grouped-query attention; the
 * "FlashAttention" page, systems-analysis.ru, section "FlashAttention-2
 * (2023)", names multi-query attention among the extensions).
 *   q, o     bf16 [B][H][N][d], lse fp32 [B][H][N], as for fa_fwd.
 *   k, v     bf16 [B][Hkv][N][d]: Hkv K/V heads, Hkv >= 1 dividing H.
 * Query head h attends with K/V head h / (H / Hkv): consecutive groups of
 * H / Hkv query heads share one K/V head (Hkv == 1 is multi-query attention,
 * Hkv == H is fa_fwd). Hkv < 1 or not dividing H -> FA_ERR_INVALID_ARG.
 * Everything else as for fa_fwd.
 */
fa_status_t fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                       hipStream_t stream);

/*
 * Forward with Nq query rows and Nk keys per head (a rectangular score
 * matrix: a chunk of new queries against a longer key sequence, or the
 * reverse). Query row i sits at sequence position Nk - Nq + i, so with
 * causal set it keeps the keys j <= Nk - Nq + i (bottom-right alignment; if
 * Nq > Nk the first Nq - Nk rows keep no key and get O = 0, lse = -inf).
 *   q, o     bf16 [B][H][Nq][d], lse fp32 [B][H][Nq].
 *   k, v     bf16 [B][Hkv][Nk][d], K/V heads shared as in fa_fwd_gqa.
 * Nq == Nk is fa_fwd_gqa. Nk < 0, or Nk == 0 with query rows to compute ->
 * FA_ERR_INVALID_ARG; Nk beyond 2^26 -> FA_ERR_UNSUPPORTED. Everything else
 * as for fa_fwd.
 */
fa_status_t fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                        hipStream_t stream);

/*
 * Forward for training: fa_fwd_rect (so also fa_fwd and fa_fwd_gqa, with
 * Nq == Nk and Hkv == H as needed) that also stores O's rounding residual.
 *   o_res    (out) bf16 [B][H][Nq][d]: o_res = bf16(O - o), with O the fp32
 *            value that o rounds. o + o_res carries O to about 16 significant
 *            bits. fa_bwd_train uses it to form D_i = dO_i . O_i without the
 *            error of o's rounding. Like lse, it is an O(N) side output kept
 *            for the backward. NULL with rows to compute -> FA_ERR_INVALID_ARG;
 *            16-byte aligned.
 * o and lse are bit for bit those of fa_fwd_rect. Everything else as for
 * fa_fwd_rect.
 */
fa_status_t fa_fwd_train(const void* q, const void* k, const void* v, void* o, void* o_res,
                         float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                         float scale, hipStream_t stream);

/*
 * Forward with 8-bit floating-point operands (the FP8 arithmetic that the
 * "FlashAttention-2" page, section "Comparison with later versions /
 * FlashAttention-3", and the "FlashAttention" page, section
 * "FlashAttention-3 (2024)", attribute to FlashAttention-3).
 *   q        (in)  e4m3 (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3
 *                  mantissa bits, no infinities) [B][H][Nq][d], one byte each;
 *                  real value = descale_q * stored value.
 *   k, v     (in)  e4m3 [B][Hkv][Nk][d], real values descale_k * k and
 *                  descale_v * v; heads shared and query rows aligned as in
 *                  fa_fwd_rect (causal: bottom-right).
 *   o        (out) bf16 [B][H][Nq][d]; lse (out) fp32 [B][H][Nq], as fa_fwd,
 *                  of attention over the real (dequantised) values.
 * Q K^T and P V run on e4m3 MFMA with fp32 accumulation; the softmax
 * statistics are fp32; the probabilities are rounded to e4m3 (scaled by 2^4)
 * only as the operand of P V, and O is normalised by the sum of those rounded
 * probabilities. d must be 128 (else FA_ERR_UNSUPPORTED); descales must be
 * finite and > 0 (else FA_ERR_INVALID_ARG). Tensor pointers 16-byte aligned.
 * Everything else as for fa_fwd_rect.
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       float descale_q, float descale_k, float descale_v, hipStream_t stream);

/*
 * Forward, fp32 storage and fp32 arithmetic throughout (no reduced-precision
 * operands). Same layout, masking, outputs and errors as fa_fwd.
 */
fa_status_t fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
                       float* lse, int B, int H, int N, int d, int causal,
                       float scale, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (0 if a size is not
 * positive or d is unsupported). The workspace is O(B*H*N*d): per row it
 * holds power-of-two-scaled fp16 copies of that row of q, dout and k (stored
 * transposed per 64-row tile) and, per query row, lse, D_i and dout_i . o_i
 * (fp32), plus a few values per head (see fa_bwd).
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/* Workspace bytes for fa_bwd_gqa (0 also when Hkv < 1 or Hkv does not divide
 * H). fa_bwd_workspace_size(B, H, N, d) equals this with Hkv == H. */
size_t fa_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d);

/*
 * Backward, bfloat16 storage: the gradients of the scalar
 * L = sum_{b,h,i,c} O_bhic dO_bhic with respect to q, k and v.
 *   q, k, v   (in)  bf16 [B][H][N][d], the forward inputs.
 *   o         (in)  bf16 [B][H][N][d], the forward output. D_i = sum_j P_ij
 *                   dP_ij = dO_i . O_i is needed for every dS, and the bf16 o
 *                   alone would move it too far (its rounding error times |dO|
 *                   reaches the 1e-2 scale of the gradients). So only a centre
 *                   D^_i = dO_i . o_i is taken from o, and the dQ pass forms D
 *                   exactly from P and dP = dO V^T (a fourth product per
 *                   score: the correction -(D - D^) sum_j P_ij k_j).
 *                   fa_bwd_train, given the forward's rounding residual of o,
 *                   forms D in the preprocess instead.
 *   dout      (in)  bf16 [B][H][N][d], dL/dO.
 *   lse       (in)  fp32 [B][H][N], the forward's logsumexp.
 *   dq,dk,dv  (out) bf16 [B][H][N][d].
 *   workspace (scratch) device buffer of at least
 *             fa_bwd_workspace_size(B, H, N, d) bytes, 256-byte aligned; its
 *             contents on entry do not matter and are overwritten.
 * P = exp(scale Q K^T - lse) is recomputed, never stored. The products that
 * form dQ, dK and dV take fp16 operands: P, dS = P * (dP - D) for dK, and
 * P * (dP - D^) for dQ (with the exact correction), against q, k, dout
 * multiplied by per-head powers of two; fp32 accumulation.
 * The result is deterministic: no floating-point atomics are used, so
 * repeated calls give identical bits. causal and scale must match the
 * forward call. The inputs must be finite.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * Backward of fa_fwd_gqa. q, o, dout, dq bf16 [B][H][N][d] and lse fp32
 * [B][H][N] as for fa_bwd; k, v, dk, dv bf16 [B][Hkv][N][d]. dk and dv of a
 * K/V head are the sums over its H / Hkv query heads (the chain rule through
 * the shared head), accumulated in a fixed order, so the result is still
 * deterministic. workspace: fa_bwd_gqa_workspace_size(B, H, Hkv, N, d) bytes.
 * Hkv < 1 or not dividing H -> FA_ERR_INVALID_ARG. Everything else as for
 * fa_bwd; fa_bwd is this with Hkv == H.
 */
fa_status_t fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                       hipStream_t stream);

/*
 * Backward of fa_fwd_rect: Nq query rows against Nk keys per head, query row
 * i at sequence position Nk - Nq + i (causal: bottom-right alignment).
 *   q, o, dout, dq  bf16 [B][H][Nq][d]; lse fp32 [B][H][Nq], fa_fwd_rect's
 *                   (rows that keep no key have lse = -inf and get dq = 0).
 *   k, v, dk, dv    bf16 [B][Hkv][Nk][d]; dk and dv of a K/V head sum over
 *                   its query heads as in fa_bwd_gqa.
 *   workspace       fa_bwd_rect_workspace_size(B, H, Hkv, Nq, Nk, d) bytes
 *                   (0 if a size is not positive, d unsupported or Hkv does
 *                   not divide H), 256-byte aligned.
 * Nq == Nk is fa_bwd_gqa. B or H == 0 (or Nq == Nk == 0) is a no-op; exactly
 * one of Nq, Nk zero, or Nk < 0 -> FA_ERR_INVALID_ARG (with no query rows
 * the gradients of k and v are zero: the library leaves them to the
 * caller); Nk beyond 2^26 -> FA_ERR_UNSUPPORTED. Everything else as for
 * fa_bwd.
 */
size_t fa_bwd_rect_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d);

fa_status_t fa_bwd_rect(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                        hipStream_t stream);

/*
 * Backward for training: fa_bwd_rect given the forward's rounding residual of
 * o (fa_fwd_train's o_res, bf16 [B][H][Nq][d], 16-byte aligned; NULL with
 * rows or keys to compute -> FA_ERR_INVALID_ARG). D_i = dO_i . (o_i + o_res_i)
 * is formed in the preprocess, where o + o_res is exact in fp32, and the dQ
 * pass takes it from there: dQ = scale sum_j P_ij (dP_ij - D_i) k_j, three
 * products per score instead of four. Same gradients within the same
 * tolerances as fa_bwd_rect (not the same bits), same workspace
 * (fa_bwd_rect_workspace_size), same determinism. Everything else as for
 * fa_bwd_rect.
 */
fa_status_t fa_bwd_train(const void* q, const void* k, const void* v, const void* o,
                         const void* o_res, const void* dout, const float* lse, void* dq,
                         void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         hipStream_t stream);

/*
 * Decoding: attention of the last Nq positions of a sequence against all of
 * its Nk keys (Nq <= Nk), the step an inference system repeats per token,
 * with the keys split into ranges whose partial results are merged with the
 * online-softmax statistics (the "FlashAttention" page, section "Online
 * softmax"; split-K/V decoding is what inference engines such as
 * FlashDecoding++ and FlashInfer, in the "FlashAttention-2" page's
 * References, do).
 *   q        (in)  bf16 [B][H][Nq][d]; row i is position Nk - Nq + i.
 *   k, v     (in)  bf16 [B][Hkv][Nk][d]; K/V heads shared as in fa_fwd_gqa.
 *   o        (out) bf16 [B][H][Nq][d]; lse (out) fp32 [B][H][Nq], as fa_fwd.
 *   causal   row i keeps keys j <= Nk - Nq + i (bottom-right alignment);
 *            otherwise every row sees all Nk keys. With Nq == 1 the two agree.
 *   workspace (scratch) fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d) bytes,
 *            256-byte aligned.
 * Limits: (H / Hkv) * Nq <= 32 (the query rows that read one K/V head are
 * packed into one 32-row block) and d in {64, 128, 256}, else
 * FA_ERR_UNSUPPORTED; Nq > Nk or Hkv not dividing H -> FA_ERR_INVALID_ARG.
 * B, H or Nq == 0 is a no-op.
 */
size_t fa_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d);

fa_status_t fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                      hipStream_t stream);

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It makes no allocation of any kind: the
 * partial results go to a fixed device buffer of the library, 40 MiB per
 * GPU, which each GPU that runs this entry point holds until the process
 * ends. Arguments, layouts, limits and results are those of fa_decode, with
 * the same kernels and the same key ranges (the output has the same bits).
 *   Limit    problems with fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d) >
 *            40 MiB (more K/V heads than the compute units hold in one round
 *            of waves, roughly B * Hkv > 1024 at d = 128) -> FA_ERR_WORKSPACE,
 *            before anything is enqueued.
 *   Sharing  every call on one GPU uses that GPU's single buffer: calls that
 *            overlap in time on one GPU (other streams, other threads) race
 *            and give wrong results. Calls on one stream are ordered and safe.
 *            Nothing in the buffer needs to be zero: each call writes every
 *            value it later reads.
 */
fa_status_t fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                              float scale, hipStream_t stream);

/*
 * The three phases of fa_bwd, for callers that schedule or time them
 * separately. fa_bwd(...) is exactly fa_bwd_preprocess (o_res NULL),
 * fa_bwd_dq (d_ready 0) and fa_bwd_dkdv, in this order, on one stream;
 * fa_bwd_train with Nq == Nk and Hkv == H is the same with o_res given and
 * d_ready 1. Each phase reads what the previous ones left in the workspace,
 * so they must run in this order. Arguments mean what they mean for fa_bwd
 * and fa_bwd_train.
 *   fa_bwd_preprocess  per-head largest magnitudes of q, k, v, dout, the
 *                      power-of-two factors derived from them, dout_i . o_i
 *                      per query row (o_i + o_res_i when o_res is given), and
 *                      the scaled fp16 transposed copies of q, dout and k ->
 *                      workspace.
 *   fa_bwd_dq          writes dq; leaves lse and D per query row in the
 *                      workspace (and, for some shapes, the scaled fp16 copies
 *                      of q and dout that the preprocess then leaves out).
 *                      d_ready must be nonzero exactly when the
 *                      preprocess of this workspace was given o_res: it
 *                      selects the pass that takes D from the workspace, and
 *                      the preprocess lays out the workspace for that pass
 *                      (a mismatch gives wrong gradients).
 *   fa_bwd_dkdv        writes dk and dv from q, k, v, dout and the workspace
 *                      (lse is taken from the workspace).
 */
fa_status_t fa_bwd_preprocess(const void* q, const void* k, const void* v, const void* o,
                              const void* o_res, const void* dout, void* workspace,
                              size_t workspace_bytes, int B, int H, int N, int d,
                              hipStream_t stream);

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* workspace, size_t workspace_bytes, void* dq,
                      int B, int H, int N, int d, int causal, float scale, int d_ready,
                      hipStream_t stream);

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
