/*
 * attn.h -- C ABI of the exact attention forward library (libattn.so).
 *
 * The library computes the exact attention forward pass
 *     S = alpha * Q K^T,  P = softmax(S) (row-wise),  O = P V
 * together with the per-row log-sum-exp LSE_i = ln sum_j exp(S_ij),
 * without ever writing the N x N matrices S or P to device memory: each
 * workgroup keeps one block of query rows on chip and streams blocks of K
 * and V through it with the online (running max m, running sum l,
 * unnormalised output O~) softmax recurrence.
 *
 * Passages defining the operations (pages on FlashAttention-3):
 *   - "FlashAttention-3 paper review" (diycv.top), problem background:
 *     S = alpha Q K^T, P = softmax(S), O = P V, alpha typically 1/sqrt(d).
 *   - "FlashAttention-3 on Hopper", section 3.1 (masks as -inf before the
 *     softmax), 3.2 and 4.2 (the online state and its invariant),
 *     4.6 (finalize: empty rows give O = 0 and LSE = -inf; LSE in natural-log
 *     units), 4.7 (causal predicate col > row + (N_k - N_q)),
 *     6.3 (block quantisation with per-tile descales), 6.4 (incoherent
 *     processing with M = H D / sqrt(d)).
 *   - "03 · FA3：Hopper 上的异步化与 overlap", section 4 (descales folded into
 *     the softmax scale; Max_offset = 8 for FP8).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layout   q, k, v, o are dense row-major [B, N, H, d] tensors (d fastest,
 *            row stride H*d elements), the logical (batch, seqlen, head, dim)
 *            order of the pages. lse is float32 [B, H, N]. N_q = N_k = N.
 *   Pointers device pointers, 16-byte aligned; the caller allocates and owns
 *            every buffer. o and lse must not overlap q, k or v.
 *   Stream   every call is asynchronous on `stream` (a hipStream_t; NULL is
 *            the default stream) and returns once its kernels are enqueued.
 *   Errors   arguments are checked on the host before anything is launched;
 *            a failing call returns a negative attn_status, launches nothing,
 *            and leaves a message readable through attn_last_error().
 *            N = 0 is a valid no-op. Nothing is printed, no exception
 *            crosses the ABI.
 *   State    the library keeps no state between calls except the
 *            thread-local error message; it allocates no device memory
 *            (attn_fwd_ex_noalloc uses a static device array instead of a
 *            caller workspace).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad alpha */
  ATTN_ERR_UNSUPPORTED = -2, /* valid request the library does not implement */
  ATTN_ERR_HIP = -3          /* the HIP runtime reported an error */
} attn_status;

typedef enum {
  ATTN_DTYPE_BF16 = 0, /* bfloat16 inputs and output */
  ATTN_DTYPE_F16 = 1   /* IEEE binary16 inputs and output */
} attn_dtype;

/*
 * attn_fwd -- exact attention forward, 16-bit inputs.
 *
 *   q, k, v  [B, N, H, d] in `dtype` (read only).
 *   o        [B, N, H, d] in `dtype` (written): O = softmax(alpha q k^T) v,
 *            each element rounded to nearest even from float32.
 *   lse      [B, H, N] float32 (written): natural-log log-sum-exp of the
 *            scaled, masked scores of each row; -inf for a row with no
 *            visible key (whose O row is then 0).
 *   B, H, N  >= 1 (N = 0 allowed: no-op).  B*N*H*d must fit in int64 and
 *            B*H*N in int32 range.
 *   d        64, 128 or 256 (other values: ATTN_ERR_UNSUPPORTED).
 *   causal   0: every key visible; 1: key j is masked for query i when j > i.
 *   alpha    softmax scale; finite and >= 0 (typically 1/sqrt(d)).
 *   dtype    an attn_dtype.
 *   stream   hipStream_t to launch on.
 *
 * Accumulation is float32; P is rounded to `dtype` before the P V product.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, float alpha, int dtype,
             void* stream);

/*
 * attn_fp8_prepare -- incoherent processing + block quantisation to e4m3.
 *
 *   x        [B, N, H, d] bfloat16 input (read only).
 *   x8       [B, N, H, d] uint8 output: OCP e4m3 (e4m3fn) codes.
 *   descale  float32 output: [B, H, ceil(N / block_rows)] when
 *            block_rows = 128, or a single float when block_rows = 0
 *            (one scale for the whole tensor).
 *   block_rows  128 (per (b, h, 128-row block) scales) or 0 (per tensor).
 *   hadamard 1: first replace each row x by x M with M = H D / sqrt(d)
 *            (H the Sylvester-ordered +-1 Hadamard matrix, D the diagonal of
 *            signs drawn from `hadamard_seed`), as for Q and K; 0: no
 *            transform (always the case for V). d must be a power of two.
 *   Scale rule: per 128-row block, scale = the smallest power of two
 *            >= amax / 448 (float32 division; at least 2^-126; 1 if
 *            amax = 0), so that the forward can apply it as an E8M0 MFMA
 *            scale; per tensor (block_rows = 0), scale = amax / 448 (1 if
 *            amax = 0). code = round-to-nearest-even e4m3 of
 *            min(|y / scale|, 448) with y's sign; descale = scale. All
 *            arithmetic is float32.
 *   Signs:   sign[i] = -1 if bit 63 of splitmix64(hadamard_seed + i) is set,
 *            else +1, where splitmix64(s) is the first output of a SplitMix64
 *            generator with state s.
 *
 * The per-tensor case (block_rows = 0) reduces over the whole tensor in two
 * kernels and needs no workspace: the second kernel recomputes the transform.
 */
int attn_fp8_prepare(const void* x, void* x8, float* descale,
                     int B, int H, int N, int d, int block_rows,
                     int hadamard, uint64_t hadamard_seed, void* stream);

/*
 * attn_fwd_fp8 -- exact attention forward on e4m3 inputs.
 *
 *   q8, k8, v8  [B, N, H, d] e4m3 codes from attn_fp8_prepare (q8 and k8
 *            prepared with the same hadamard flag and seed; v8 without the
 *            transform). Because (Q M)(K M)^T = Q K^T, the forward needs no
 *            knowledge of M.
 *   descale_q/k/v  float32 descales as written by attn_fp8_prepare with the
 *            same block_rows. With block_rows = 128, descale_v must hold
 *            powers of two (as attn_fp8_prepare writes them): the kernel
 *            applies only their exponent, as the E8M0 scale of the PV
 *            product (the "descale folded into the O rescale" of the pages,
 *            without any rescale).
 *   o        [B, N, H, d] bfloat16 output; lse [B, H, N] float32.
 *   block_rows  128 or 0, matching the descales.
 *   hadamard_seed  the seed q8 and k8 were prepared with (attn_fp8_prepare,
 *            hadamard = 1); any value when they were prepared without the
 *            transform. It is a contract, not an input to the arithmetic:
 *            Q and K must share one M for (Q M)(K M)^T = Q K^T to hold
 *            ("FlashAttention-3 on Hopper", section 6.4), the forward never
 *            applies M, and the codes do not record which M was used, so a
 *            mismatch cannot be detected and gives wrong scores.
 *   Other arguments as attn_fwd (d = 64, 128 or 256). The descales must not
 *   overlap o or lse.
 *
 * Scores are accumulated in float32 and multiplied by alpha * dq * dk per
 * tile; P is formed as exp2 of the score minus a reference that trails the
 * row maximum by at most 4.8, plus an offset of 4 (the pages' Max_offset,
 * lowered from 8 so that P <= 2^8.8 < 448 stays inside e4m3), rounded to
 * e4m3 for the P V product, which applies dv as the V operand's scale.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float alpha,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 int block_rows, uint64_t hadamard_seed, void* stream);

/*
 * attn_fwd_fp8_ex -- attn_fwd_fp8 with grouped key/value heads ("FlashAttention-3
 * on Hopper", section 5.6.1: GQA/MQA).
 *
 *   q8       [B, N, Hq, d] e4m3; o [B, N, Hq, d] bfloat16; lse [B, Hq, N].
 *   k8, v8   [B, N, Hkv, d] e4m3; query head h reads key/value head
 *            h / (Hq / Hkv). Hq must be a positive multiple of Hkv (Hkv = 1 is
 *            multi-query attention).
 *   descale_q  as written by attn_fp8_prepare for q8 (H = Hq);
 *   descale_k/v as written by attn_fp8_prepare for k8 and v8 (H = Hkv).
 *   Hkv is checked before an empty problem returns (as in attn_fwd_ex).
 *   Other arguments, layouts and errors as attn_fwd_fp8, which is this call
 *   with Hkv = Hq.
 */
int attn_fwd_fp8_ex(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, float alpha,
                    const float* descale_q, const float* descale_k, const float* descale_v,
                    int block_rows, uint64_t hadamard_seed, void* stream);

/*
 * attn_bwd -- gradients of the exact attention forward ("FlashAttention-3 on
 * Hopper", chapter 7, section 7.1): for O = softmax(alpha Q K^T) V and an
 * upstream gradient dO,
 *   D_i = rowsum(dO_i o O_i)            (section 7.1.2, written to delta)
 *   P   = exp(alpha Q K^T - LSE)        (section 7.1.3, recomputed, never stored)
 *   dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
 *   dQ  = alpha dS K,  dK = alpha dS^T Q.
 *
 *   q, k, v, o, dout  [B, N, H, d], dtype as attn_fwd (o and lse are the
 *            forward's outputs for the same q, k, v, causal, alpha).
 *   lse      [B, H, N] float32 from attn_fwd.
 *   dq, dk, dv  [B, N, H, d] outputs in the input dtype (device memory).
 *   delta    [B, H, N] float32 workspace owned by the caller; the call writes
 *            D into it (no allocation inside the library).
 *   d        64, 128 or 256 (at 256 the dK/dV kernel runs twice, once per
 *            output, recomputing S, because one wave cannot hold K, V and both
 *            accumulators).
 *   Other arguments and the error behaviour as attn_fwd. dq, dk, dv and delta
 *   must not overlap each other or the inputs.
 *
 * dQ comes from a second, query-parallel kernel that recomputes P and dP
 * (one of the pages' options for the dQ reduction, section 7.2.3), so no
 * atomics are used and the result is deterministic.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float alpha,
             int dtype, void* stream);

/*
 * attn_fwd_ex -- the 16-bit forward of attn_fwd, generalised for serving:
 * grouped / multi-query heads, N_q != N_k, packed variable-length batches,
 * and split-KV (Flash-Decoding) with a combine kernel.
 *
 *   Heads    Hq query heads over Hkv key/value heads (Hq % Hkv == 0); query
 *            head h reads key/value head floor(h / (Hq / Hkv))
 *            ("FlashAttention-3 on Hopper", section 5.6.1). Hkv = 1 is MQA.
 *   Dense    cu_seqlens_q = cu_seqlens_k = NULL: q, o are [B, Nq, Hq, d],
 *            k, v are [B, Nk, Hkv, d], lse is float32 [B, Hq, Nq];
 *            total_q and total_k are ignored.
 *   Packed   cu_seqlens_q, cu_seqlens_k: device int32 arrays of B + 1 row
 *            offsets (sequence b owns rows cu[b] .. cu[b+1]-1; the pages
 *            list variable-length batches in chapter 9.3, whose text is
 *            missing): q, o are [total_q, Hq, d], k, v are [total_k, Hkv, d],
 *            lse is float32 [Hq, total_q]. Nq and Nk are the largest sequence
 *            lengths (they size the grid; longer sequences are cut to them).
 *            Offsets are clamped into [0, total] on the device, so malformed
 *            arrays never address outside the tensors, but rows that no valid
 *            sequence covers are left unspecified.
 *   causal   1: query i of a sequence sees key j iff j <= i + (N_k - N_q)
 *            (bottom-right alignment, section 4.7); a row that sees no key
 *            gets O = 0 and LSE = -inf. With N_q = 1 this is every key.
 *   window_left, window_right  local (sliding-window) attention, >= -1:
 *            query i sees key j iff i + off - window_left <= j and
 *            j <= i + off + window_right, off = N_k - N_q; -1 leaves that side
 *            unbounded (-1, -1: no window). causal = 1 sets the right width
 *            to 0. Section 4.7 names the left boundary of local attention
 *            without a formula; this is the plainest reading with the
 *            causal alignment.
 *   pack_gqa 1: the g = Hq / Hkv query heads of one key/value head share a
 *            128-row query tile (rows interleave as query-major, head-minor),
 *            so a K/V tile is read once for the group; 0: one query head per
 *            tile; -1: attn_pack_gqa_heuristic decides. The pages list this as
 *            PackGQA (chapter 11, text missing). The result does not depend on
 *            the choice. When Nq * g <= 16 and d <= 128 (decode) a kernel for
 *            few rows runs instead, which always packs the group and ignores
 *            pack_gqa.
 *   num_splits  >= 1. With more than one range the keys are cut into
 *            consecutive ranges of split_len = 64 * ceil(ceil(Nk / num_splits)
 *            / 64) keys (the last may be shorter; empty ranges are dropped, so
 *            at most num_splits are used). Each range writes its normalised
 *            state O_s = O~_s / l_s, LSE_s = m_s + ln l_s to the workspace
 *            (float32 [S, total_q, Hq, d] then [S, total_q, Hq], S the ranges
 *            used; total_q = B * Nq for dense inputs) and a second kernel
 *            merges them, LSE = ln sum_s e^(LSE_s), O = sum_s e^(LSE_s - LSE)
 *            O_s (the block-combine rule, section 3.2.1; split-KV, chapter 10).
 *   workspace  caller-owned device memory of at least
 *            attn_splitkv_workspace_bytes(num_splits, total_q, Hq, d) bytes,
 *            16-byte aligned, not overlapping any other argument; unused (may
 *            be NULL) when one range is used.
 *   k and v may be NULL when no sequence has keys (total_k = 0, or Nk = 0
 *   for dense inputs). Other arguments, errors and the rounding as attn_fwd.
 *   Empty problems
 *   (B, Hq, Nq or total_q = 0) are no-ops; Nk = 0 (or an empty key sequence)
 *   gives O = 0 and LSE = -inf for its rows.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Nq, int Nk, int d,
                const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q, int total_k,
                int causal, int window_left, int window_right, float alpha, int dtype,
                int pack_gqa, int num_splits, float* workspace, int64_t workspace_bytes,
                void* stream);

/* Workspace bytes attn_fwd_ex needs for num_splits key ranges (0 for
 * num_splits <= 1): num_splits * total_q * Hq * (d + 1) * 4. */
int64_t attn_splitkv_workspace_bytes(int num_splits, int total_q, int Hq, int d);

/*
 * attn_fwd_ex_noalloc -- attn_fwd_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without workspace / workspace_bytes.
 * With several key ranges the range states go to a static device array the
 * library holds on each GPU (ATTN_STATIC_WORKSPACE_BYTES = 16 MiB, resident
 * from the first such call on that GPU until the process ends); the call
 * itself allocates nothing (no hipMalloc, no hipFree).
 *
 *   Limit    attn_splitkv_workspace_bytes(ranges used, total_q, Hq, d) must
 *            be <= ATTN_STATIC_WORKSPACE_BYTES, else ATTN_ERR_UNSUPPORTED
 *            (checked before any launch). One range needs no workspace.
 *   Sharing  every call on one GPU uses that GPU's single array, which keeps
 *            the last call's contents (nothing in it needs to start at
 *            zero: each range writes its whole state before the combine
 *            reads it). Calls that overlap in time on one GPU (on different
 *            streams, or from different threads) race on it; callers must
 *            order them (one stream, or events).
 *   Device   the array of the current device (hipGetDevice) is used; the
 *            stream must belong to that device.
 *   Result   identical to attn_fwd_ex with the same arguments (same kernels).
 */
#define ATTN_STATIC_WORKSPACE_BYTES (16 << 20)
int attn_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q, int total_k,
                        int causal, int window_left, int window_right, float alpha, int dtype,
                        int pack_gqa, int num_splits, void* stream);

/* 1 if packing the query heads of a group takes fewer 128-row query tiles
 * than one head per tile (e.g. decode with Nq = 1 and Hq > Hkv), else 0. */
int attn_pack_gqa_heuristic(int Hq, int Hkv, int Nq);

/* Suggested num_splits for attn_fwd_ex on a device with num_cus compute
 * units. With Nq * Hq / Hkv <= 16 query rows per key/value head and d <= 128
 * (decode) the call runs a kernel with one workgroup per (sequence,
 * key/value head, range): enough ranges for about num_cus workgroups, at
 * least 512 keys each. Otherwise: 1 when the 128-row query tiles alone fill
 * every resident workgroup slot (two per compute unit for d <= 128, one for
 * d = 256), else enough ranges to fill them, at least 256 keys each. At most
 * 128 ranges. pack_gqa as in attn_fwd_ex. */
int attn_num_splits_heuristic(int B, int Hq, int Hkv, int Nq, int Nk, int d, int pack_gqa, int num_cus);

/*
 * attn_bwd_ex -- attn_bwd generalised like attn_fwd_ex: Hq query heads over
 * Hkv key/value heads, N_q != N_k, packed variable-length batches and local
 * (sliding-window) attention.
 *
 *   Dense    cu_seqlens_q = cu_seqlens_k = NULL: q, o, dout, dq are
 *            [B, Nq, Hq, d]; k, v, dk, dv are [B, Nk, Hkv, d]; lse, delta are
 *            float32 [B, Hq, Nq]; total_q and total_k are ignored.
 *   Packed   device int32 cu_seqlens_q, cu_seqlens_k of B + 1 row offsets, as
 *            in attn_fwd_ex: q, o, dout, dq are [total_q, Hq, d]; k, v, dk, dv
 *            are [total_k, Hkv, d]; lse, delta are float32 [Hq, total_q].
 *            Nq, Nk are the largest sequence lengths. Rows that no valid
 *            sequence covers are left unspecified in dq, dk, dv and delta.
 *   causal, window_left, window_right  the mask of the forward call that
 *            produced o and lse (same meaning as in attn_fwd_ex).
 *   The gradient of key/value head kh is the sum over the Hq / Hkv query
 *   heads that read it ("FlashAttention-3 on Hopper", section 8.8): each
 *   dK/dV workgroup loops over those heads' query tiles itself, so the sum
 *   takes no atomics and the result is deterministic. Masked keys and
 *   queries get zero gradients: a sequence with no query rows writes zero
 *   dK, dV, one with no key rows zero dQ; the pointers of operands of size
 *   zero may then be NULL. Other arguments and errors as attn_bwd.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q, int total_k,
                int causal, int window_left, int window_right, float alpha, int dtype, void* stream);

/* Message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char* attn_last_error(void);

/* Library version string: "attn-gfx950 <version> (commit <c>, hip <v>, rocm
 * <r>, <arch>)", the provenance recorded when the library was built. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
