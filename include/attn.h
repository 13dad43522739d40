/*
 * attn.h -- C ABI of the MI355X (gfx950) attention forward library, libattn.so.
 *
 * The library computes, for every batch b, head h and query row i,
 *
 *     O[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:] ) V[b,h,j,:]
 *     LSE[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,h,j,:] )
 *
 * with the causal option removing every key j > i before the softmax (top-left
 * aligned: row i sees keys 0..i). Sources: "Flash Attention 4 -- the algorithm
 * and the two-MMA problem" (the attention formula, the online-softmax update and
 * deferred normalisation, the exp2 fold); "Lecture 2 -- Online Softmax and
 * Numerical Correctness" (safe softmax, the LSE side output, the causal rule);
 * "FlashAttention-4's Softmax Tricks" (the lagging-max threshold tau and the
 * degree-3 software exp2). S and P are never written to memory: the kernels
 * stream K and V in tiles with a running max, denominator and accumulator.
 *
 * Conventions for every entry point
 *   - Pointers named Q, K, V, O, LSE, *_scale, x, y are DEVICE pointers (HIP
 *     device memory, e.g. from torch). The caller owns all memory; the library
 *     allocates nothing and keeps no state between calls except the thread-local
 *     error message.
 *   - Layout: Q [B,H,Nq,d], K and V [B,H,Nk,d], O [B,H,Nq,d], all contiguous with
 *     d innermost. LSE [B,H,Nq] float32. Every tensor pointer must be 16-byte
 *     aligned.
 *   - Launches are asynchronous on the given stream (NULL = the null stream);
 *     no call synchronises. On success every element of O and LSE has been
 *     written once the stream reaches that point.
 *   - Validation happens before any HIP call; on a validation error nothing is
 *     launched and nothing is written. A non-zero status leaves a message for
 *     attn_last_error().
 *   - Reentrant: concurrent calls on different streams are independent.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (0 = success, negative = error). */
enum {
  ATTN_OK = 0,
  ATTN_E_NULLPTR = -1,   /* a required pointer is NULL                               */
  ATTN_E_SHAPE = -2,     /* B, H, Nq < 0; Nk < 1 with work to do; sizes too large
                            (Nq or Nk above 2^30, or one (b, h) slice of Q, K or V
                            of 2 GiB or more); MXFP8 with Nq or Nk not a
                            multiple of 32                                            */
  ATTN_E_HEADDIM = -3,   /* d not supported for the dtype (bf16: 64, 128, 192 or
                            256; f32: 64 or 128; MXFP8: 128)                           */
  ATTN_E_DTYPE = -4,     /* unknown dtype code                                         */
  ATTN_E_EXP2MODE = -5,  /* unknown exp2_mode                                          */
  ATTN_E_TAU = -6,       /* tau negative, above 64 or not finite; for the fixed-scale
                            FP8 P dtypes, 8 + tau >= log2 of P's largest finite value
                            (448 for E4M3, 57344 for E5M2)                             */
  ATTN_E_SCALE = -7,     /* scale not finite or <= 0                                   */
  ATTN_E_ALIGN = -8,     /* a tensor pointer is not 16-byte aligned (MX scale pointers:
                            4-byte aligned)                                            */
  ATTN_E_HIP = -9        /* a HIP launch failed (message has the HIP error string)     */
};

/* Input dtypes. O is float32 for ATTN_F32 and bf16 for ATTN_BF16 and MXFP8. */
enum {
  ATTN_F32 = 0,          /* Q, K, V, O float32                                         */
  ATTN_BF16 = 1,         /* Q, K, V, O bfloat16                                        */
  ATTN_MXFP8_E4M3 = 2,   /* Q, K, V OCP e4m3 bytes plus one E8M0 scale byte per 32x32
                            block ([B,H,N/32,d/32] uint8, V blocked along the sequence
                            with the same square blocks); O bfloat16. Source: "PyTorch
                            FlashAttention-4 adds MXFP8 block-scaled forward and backward
                            for Blackwell", section "Quantization along both axes and
                            jagged tensors". P is re-quantised to e4m3 per 32 keys
                            with an E8M0 scale from that block's score maximum        */
  ATTN_MXFP8_E4M3_PFIX_E4M3 = 3,
                         /* the same inputs, but P is multiplied by 2^max_offset
                            (max_offset = 8) and cast to E4M3 with one fixed scale, as
                            FA4's FP8 path does ("FlashAttention-4's Softmax Tricks",
                            section "Where 'exact' breaks: P in FP8"); a lagging max
                            lets P reach 2^tau, so tau < log2(448) - 8 (about 0.807)
                            is required (ATTN_E_TAU otherwise)                         */
  ATTN_MXFP8_E4M3_PFIX_E5M2 = 4
                         /* as ATTN_MXFP8_E4M3_PFIX_E4M3 with P cast to E5M2 (largest
                            finite 57344): tau < log2(57344) - 8 (about 7.807)          */
};

/*
 * exp2 of the per-score probabilities P = 2^(S*scale*log2(e) - m*scale*log2(e)):
 *   ATTN_EXP2_HW   the hardware exponential (v_exp_f32)
 *   ATTN_EXP2_EMU  the degree-3 software exp2 for every P ("FlashAttention-4's
 *                  Softmax Tricks", section "The emulated exp2": clamp at -127,
 *                  split into floor and fraction, 3-FMA Horner polynomial, integer
 *                  add of floor into the exponent bits)
 *   ATTN_EXP2_MIX  a fixed share of each lane's P through the software exp2 and the
 *                  rest through the hardware one; the share comes from the library's
 *                  tuning table keyed by (dtype, d, causal)
 *   ATTN_EXP2_MIX_BASE + k (k = 0..16)  the same with exactly k of every 16 P
 *                  emulated (for tuning sweeps)
 *   ATTN_EXP2_EMU4, ATTN_EXP2_EMU5  every P through the software exp2 with a
 *                  degree-4 / degree-5 polynomial (same section's error table:
 *                  max relative error 3.05e-6 / 1.44e-7 against 8.77e-5 at degree
 *                  3; the page prints no coefficients, the library's are a fit of
 *                  the same kind: relative-error minimax, p0 = 1, float32).
 *                  ATTN_F32 and ATTN_BF16 only (ATTN_E_EXP2MODE for MXFP8).
 * The rescale factor and the LSE logarithm always use the hardware units.
 */
enum {
  ATTN_EXP2_HW = 0,
  ATTN_EXP2_EMU = 1,
  ATTN_EXP2_MIX = 2,
  ATTN_EXP2_EMU4 = 3,
  ATTN_EXP2_EMU5 = 4,
  ATTN_EXP2_MIX_BASE = 16
};

/*
 * attn_fwd -- bf16 attention forward on the null stream.
 *
 *   Q, K, V   device bf16, [B,H,Nq,d] / [B,H,Nk,d] / [B,H,Nk,d]
 *   O         device bf16 [B,H,Nq,d] (written)
 *   LSE       device float32 [B,H,Nq] (written): natural-log log-sum-exp of the
 *             scaled scores of each row
 *   B, H, Nq  >= 0 (a zero means there is nothing to do: returns ATTN_OK)
 *   Nk        >= 1 when B*H*Nq > 0
 *   d         64, 128, 192 or 256
 *   causal    0 = no mask; 1 = causal aligned top-left: key j is removed for
 *             query i when j > i ("Lecture 2 -- Online Softmax and Numerical
 *             Correctness", section "Causal masking just changes which blocks
 *             contribute"); 2 = causal aligned bottom-right: removed when
 *             j > i + Nk - Nq, so the last query sees every key (the same mask as
 *             1 when Nq == Nk). A row that sees no key (2 with Nq > Nk) gets
 *             O = 0 and LSE = -inf.
 *   scale     > 0 and finite; multiplies Q.K (1/sqrt(d) for standard attention)
 *   exp2_mode ATTN_EXP2_* above
 *   tau       lagging-max threshold in log2 units of the scaled scores
 *             ("FlashAttention-4's Softmax Tricks", section "Conditional
 *             rescaling, and when it's exact"): O and the denominator are rescaled
 *             only when the row max grows by more than tau; 0 <= tau <= 64
 *             (P stays below 2^tau, far inside float32 and bf16 range)
 */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
             int B, int H, int Nq, int Nk, int d, int causal, float scale,
             int exp2_mode, float tau);

/*
 * attn_fwd_ex -- attn_fwd with an explicit dtype, MX scales and stream.
 *
 *   dtype     ATTN_F32, ATTN_BF16, ATTN_MXFP8_E4M3, ATTN_MXFP8_E4M3_PFIX_E4M3 or
 *             ATTN_MXFP8_E4M3_PFIX_E5M2
 *   q_scale, k_scale, v_scale
 *             device uint8 E8M0 bytes, [B,H,Nq/32,d/32] and [B,H,Nk/32,d/32];
 *             required for the three MXFP8 dtypes, ignored (may be NULL) otherwise
 *   stream    a hipStream_t (e.g. torch.cuda.current_stream().cuda_stream), or NULL
 * For ATTN_MXFP8_E4M3, P is re-quantised to e4m3 per 32 keys with an E8M0 scale
 * taken from that block's score maximum, so a lagging max cannot saturate P (the
 * failure "FlashAttention-4's Softmax Tricks" describes in "Where 'exact' breaks:
 * P in FP8" needs a fixed P scale); tau = 0, the setting that page gives for FP8,
 * is the usual choice. The two PFIX dtypes use that fixed scale and therefore
 * bound tau by the P format's range.
 */
int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
                int B, int H, int Nq, int Nk, int d, int causal, float scale,
                int exp2_mode, float tau, int dtype,
                const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                void* stream);

/*
 * attn_fwd_split_workspace_bytes -- bytes of float32 workspace attn_fwd_split
 * needs for this launch: 0 when the launch is not split (dtype other than
 * ATTN_BF16, nothing to compute, or key_chunk = 0 and the library runs the
 * launch whole); -1 when the sizes or key_chunk are invalid (as attn_fwd_ex
 * would reject them).
 */
long long attn_fwd_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal,
                                         int dtype, int key_chunk);

/*
 * attn_fwd_split -- attn_fwd_ex that may cut each row's keys into chunks run
 * by separate workgroups, for launches with too few query tiles to fill the
 * GPU (small batches, few heads, decoding-like Nq << Nk).
 *
 * Source: "Lecture 2 -- Online Softmax and Numerical Correctness", section
 * "Combining two blocks exactly": the softmax states (max, denominator,
 * output) of two key ranges combine exactly into the state of their union,
 * so a row may be computed chunk by chunk anywhere and merged afterwards.
 * Each chunk's workgroup writes its normalised float32 output O_k and its
 * log-sum-exp L_k (log2 units) to the workspace; a second kernel forms
 * L = max L_k, w_k = 2^(L_k - L), O = sum w_k O_k / sum w_k and
 * LSE = ln2 * (L + log2 sum w_k). Query tiles whose keys fit one chunk are
 * written directly.
 *
 *   Q .. stream   as attn_fwd_ex (all dtypes; only ATTN_BF16 dense launches
 *                 are split, every other launch runs as attn_fwd_ex and
 *                 needs no workspace)
 *   key_chunk     0: the library's choice: a launch is split when run whole
 *                 it would occupy fewer than a quarter of the compute units
 *                 (decoding-like shapes, few heads), or, for d = 128 launches
 *                 small enough for the key-parity kernel, at most half of
 *                 them with rows of 32 or more key-tile steps; into chunks of
 *                 at least 128 keys sized for two workgroups per compute
 *                 unit; larger launches run whole (measured: splitting gains
 *                 nothing there, the partials' memory traffic costs what the
 *                 shorter chains save);
 *                 > 0: a multiple of 64, keys per chunk (bf16 launches are
 *                 then always run by the split kernels)
 *   workspace     device memory of >= attn_fwd_split_workspace_bytes(...)
 *                 bytes, 16-byte aligned, owned by the caller (NULL allowed
 *                 when that size is 0); contents on entry are ignored and
 *                 nothing in it needs to start at zero. Calls that share a
 *                 workspace must not overlap.
 *   workspace_bytes  its size
 * Exp2 modes, tau and the causal settings are those of attn_fwd_ex; the
 * rescale decisions of the lagging max are taken per chunk. Errors: those of
 * attn_fwd_ex; ATTN_E_SHAPE for a bad key_chunk or a workspace that is too
 * small, ATTN_E_NULLPTR / ATTN_E_ALIGN for a missing or unaligned workspace.
 */
int attn_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int Nq, int Nk, int d, int causal, float scale,
                   int exp2_mode, float tau, int dtype,
                   const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                   int key_chunk, float* workspace, long long workspace_bytes, void* stream);

/* Bytes of the device scratch array attn_fwd_split_noalloc uses (64 MiB). */
enum { ATTN_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024 };

/*
 * attn_fwd_split_noalloc -- attn_fwd_split for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The call allocates nothing (no hipMalloc, no library
 * routine that allocates); the split launch's workspace is a file-scope
 * device array of ATTN_NOALLOC_SCRATCH_BYTES bytes that every device the
 * library runs on holds from load until the process ends.
 *
 *   arguments     those of attn_fwd_split without the workspace
 *   key_chunk     0: the library's choice, with the chunk doubled as often as
 *                 needed for the partials to fit the scratch (or the launch
 *                 run whole); > 0: a multiple of 64 whose partials must fit,
 *                 else ATTN_E_SHAPE
 *   stream        must belong to the current device (ATTN_E_HIP otherwise);
 *                 the scratch address of each device is looked up once, on
 *                 the first call made with that device current
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents: calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller. Nothing in the scratch
 * needs to start at zero. Results equal attn_fwd_split's for the same
 * key_chunk. Errors: those of attn_fwd_split.
 */
int attn_fwd_split_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int B, int H, int Nq, int Nk, int d, int causal, float scale,
                           int exp2_mode, float tau, int dtype,
                           const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                           int key_chunk, void* stream);

/*
 * attn_fwd_varlen -- a batch of sequences of different lengths, packed.
 *
 *   Q, O      device [total_q, H, d] (token-major: row t of head h at (t*H + h)*d)
 *   K, V      device [total_k, H, d]
 *   LSE       device float32 [H, total_q] (written)
 *   cu_seqlens_q, cu_seqlens_k
 *             device int32 arrays of B+1 entries: sequence b owns query rows
 *             cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 *             cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (non-decreasing, starting at 0,
 *             ending at total_q / total_k). Each sequence is one attention problem
 *             with its own Nq and Nk; causal alignment (1 = top-left, 2 =
 *             bottom-right) applies per sequence. A sequence with no keys gets
 *             O = 0 and LSE = -inf. Offsets outside [0, total] are clamped, so
 *             inconsistent arrays shorten sequences but never move an access
 *             outside the tensors.
 *   max_seqlen_q  >= every query length (query tiles past it are not computed)
 *   dtype     ATTN_F32 or ATTN_BF16 (MXFP8 batches carry scales: attn_fwd_varlen_ex);
 *             other arguments as for attn_fwd.
 * The kernels are those of attn_fwd_ex; only the addressing of each (sequence,
 * head) slice differs. Source for the method: as attn_fwd. Validation that
 * needs the lengths themselves cannot be done on the host (they live on the
 * device); every other check happens before any launch.
 */
int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                    int max_seqlen_q, int total_q, int total_k, int d, int causal,
                    float scale, int exp2_mode, float tau, int dtype, void* stream);

/*
 * attn_fwd_varlen_ex -- attn_fwd_varlen for every dtype, including packed MXFP8
 * batches with split-addressed scale tensors.
 *
 * Source: "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and
 * backward for Blackwell", section "Quantization along both axes and jagged
 * tensors": with jagged sequences the FP8 data stays compact and only the
 * scale tensors are laid out (padded) for the kernel.
 *
 *   Q, K, V, O, LSE, cu_seqlens_q, cu_seqlens_k, B, H, max_seqlen_q, total_q,
 *   total_k, d, causal, scale, exp2_mode, tau
 *             as attn_fwd_varlen (Q, K, V are e4m3 bytes for MXFP8; O is bf16)
 *   q_scale   device E8M0 bytes [scale_rows_q, H, d/32]: scale row
 *             scale_offsets_q[b] + r, head h, byte c scales query rows
 *             cu_seqlens_q[b] + 32r .. +31 (those inside the sequence) and
 *             elements 32c .. 32c+31 of head h. Blocks start at each
 *             sequence's first token, so a sequence's last block may be partial.
 *   k_scale, v_scale
 *             the same for K and V with scale_offsets_k and scale_rows_k
 *   scale_offsets_q, scale_offsets_k
 *             device int32 [B+1]: first scale row of each sequence (the rows
 *             between ceil(len/32) and the next sequence's offset are padding
 *             and are not read). attn_mx_scale_offsets writes them for the
 *             compact (align 32) or a padded layout. Clamped to
 *             [0, scale_rows]; blocks past scale_rows read as scale 1.
 *   scale_rows_q, scale_rows_k   rows of the scale tensors (>= 0)
 *   dtype     ATTN_F32, ATTN_BF16 or one of the MXFP8 codes; for F32/BF16 the
 *             scale arguments are ignored and may be NULL / 0
 * MXFP8 supports d = 128. Errors as attn_fwd_varlen; additionally
 * ATTN_E_NULLPTR for a missing MXFP8 scale or offset pointer and ATTN_E_ALIGN
 * for one that is not 4-byte aligned.
 */
int attn_fwd_varlen_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
                       const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                       const int* cu_seqlens_q, const int* cu_seqlens_k,
                       const int* scale_offsets_q, const int* scale_offsets_k,
                       int scale_rows_q, int scale_rows_k, int B, int H, int max_seqlen_q,
                       int total_q, int total_k, int d, int causal, float scale, int exp2_mode,
                       float tau, int dtype, void* stream);

/*
 * attn_mx_scale_offsets -- first scale row of each packed sequence.
 *
 * Source: as attn_fwd_varlen_ex (the scale tensors of a jagged batch are
 * padded to aligned positions while the data stays compact).
 *
 *   cu_seqlens  device int32 [B+1] sequence starts (clamped to [0, total])
 *   align       rows of sequence alignment, a multiple of 32 in [32, 4096]:
 *               32 gives the compact layout, 128 the page's padded one
 *   offsets     device int32 [B+1] (written): offsets[b] = sum over b' < b of
 *               ceil(len(b') / align) * align / 32; offsets[B] is the number
 *               of scale rows the layout needs
 * One small kernel on `stream`; ATTN_E_SHAPE when the row count could
 * overflow int32, ATTN_E_NULLPTR / ATTN_E_ALIGN for bad pointers.
 */
int attn_mx_scale_offsets(const int* cu_seqlens, int B, int total, int align, int* offsets,
                          void* stream);

/*
 * attn_mx_scale_scatter -- copy packed MXFP8 scales from one layout into
 * another (e.g. compact jagged into 128-aligned padded rows).
 *
 * Source: as attn_fwd_varlen_ex (the scatter/layout kernels that move scales
 * from the compact jagged layout into the padded one).
 *
 *   src, dst    device E8M0 bytes [src_rows, H, d/32] / [dst_rows, H, d/32]
 *   src_offsets, dst_offsets
 *               device int32 [B+1] first scale row of each sequence
 *   cu_seqlens  device int32 [B+1] sequence starts (clamped to [0, total])
 * Destination rows dst_offsets[b] .. dst_offsets[b+1]-1 (clamped to
 * [0, dst_rows]) receive sequence b's ceil(len/32) rows from src_offsets[b]
 * in order; the rest of that range, and rows whose source lies outside
 * [0, src_rows), are set to 127 (scale 1). dst must not overlap src.
 * d = 128 only (ATTN_E_HEADDIM otherwise); pointers 4-byte aligned.
 */
int attn_mx_scale_scatter(const uint8_t* src, const int* src_offsets, int src_rows, uint8_t* dst,
                          const int* dst_offsets, int dst_rows, const int* cu_seqlens, int B,
                          int total, int H, int d, void* stream);

/*
 * attn_bwd_workspace_bytes -- bytes of float32 workspace attn_bwd needs:
 * 8 * B * H * Nq (two floats per query row); -1 for negative sizes.
 */
long long attn_bwd_workspace_bytes(int B, int H, int Nq);

/*
 * attn_bwd -- attention backward: dQ, dK, dV from dO and the forward pass's
 * O and LSE.
 *
 * Source: "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and
 * backward for Blackwell", section "TMEM allocation and scale factor
 * placement" (five products; dK and dV accumulate over the whole pass), and
 * "Lecture 2 -- Online Softmax and Numerical Correctness", section "Use it in
 * the real stack" (the forward pass's LSE rebuilds P, which is what makes the
 * backward pass cheap). With P = exp(scale * Q K^T - LSE) (masked as in
 * attn_fwd): dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
 * dQ = scale * dS K, dK = scale * dS^T Q.
 *
 *   Q, O, dO       device bf16 [B, H, Nq, d];  K, V: device bf16 [B, H, Nk, d]
 *   LSE            device float32 [B, H, Nq], natural log, as attn_fwd writes it
 *                  (-inf for a row that saw no key: that row gets dQ = 0 and
 *                  adds nothing to dK, dV)
 *   dQ             device bf16 [B, H, Nq, d] (written)
 *   dK, dV         device bf16 [B, H, Nk, d] (written; keys no query sees get 0)
 *   workspace      device, >= attn_bwd_workspace_bytes(B, H, Nq) bytes, owned
 *                  by the caller; holds per-row LSE*log2(e) and D between the
 *                  three kernels of one call (contents on entry are ignored)
 *   workspace_bytes  its size
 *   d              64 or 128;  causal 0, 1 (top-left) or 2 (bottom-right)
 *   scale          the forward pass's scale (> 0, finite)
 *   dtype          ATTN_BF16
 *   stream         hipStream_t (NULL = the null stream); asynchronous
 * Tensors with no elements may be NULL (Nq = 0: Q, O, dO, LSE, dQ, workspace;
 * Nk = 0: K, V, dK, dV). All pointers 16-byte aligned. Errors: ATTN_E_DTYPE,
 * ATTN_E_SHAPE (negative or too large sizes, workspace too small, causal not
 * 0..2), ATTN_E_HEADDIM, ATTN_E_SCALE, ATTN_E_NULLPTR, ATTN_E_ALIGN,
 * ATTN_E_HIP; every check happens before any launch. Calls that share a
 * workspace must not overlap.
 */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
             long long workspace_bytes, int B, int H, int Nq, int Nk, int d, int causal,
             float scale, int dtype, void* stream);

/*
 * attn_bwd_ex -- attn_bwd for ATTN_BF16 and ATTN_MXFP8_E4M3.
 *
 * Source: as attn_bwd, and "PyTorch FlashAttention-4 adds MXFP8 block-scaled
 * forward and backward for Blackwell", section "Quantization along both axes
 * and jagged tensors": the backward products reduce along both axes, so Q, K,
 * V and dO are quantised in square 32x32 blocks (one e4m3 payload serves a
 * product and its transpose), and dS likewise, so that dK and dQ consume the
 * same representation.
 *
 * ATTN_MXFP8_E4M3 (d = 128; Nq, Nk multiples of 32):
 *   Q, K, V, dO    e4m3 bytes [B, H, N, 128]
 *   q_scale, k_scale, v_scale, do_scale
 *                  E8M0 bytes [B, H, N/32, 4], one per 32x32 block (those of
 *                  attn_fwd_ex for Q, K, V; attn_mx_quantize writes dO's)
 *   O              bf16 [B, H, Nq, 128] as attn_fwd_ex wrote it; LSE float32
 *   dQ, dK, dV     bf16 (written)
 * Inside, P is stored times 2^8 with one fixed scale (P <= 1: the LSE is
 * exact) and dS with one E8M0 byte per 32x32 block from its amax.
 * Other arguments and errors as attn_bwd; additionally ATTN_E_SHAPE for MXFP8
 * sizes that are not multiples of 32, ATTN_E_NULLPTR / ATTN_E_ALIGN for
 * missing or unaligned (4-byte) scale pointers. For ATTN_BF16 the scale
 * pointers are ignored.
 */
int attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                long long workspace_bytes, int B, int H, int Nq, int Nk, int d, int causal,
                float scale, int dtype, const uint8_t* q_scale, const uint8_t* k_scale,
                const uint8_t* v_scale, const uint8_t* do_scale, void* stream);

/*
 * attn_mx_quantize -- bf16 [rows, 128] to e4m3 [rows, 128] with one E8M0 byte
 * per square 32x32 block ([rows/32, 4]), the layout attn_fwd_ex and
 * attn_bwd_ex read (pass rows = B*H*N with N a multiple of 32).
 *
 * Source: "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and
 * backward for Blackwell", section "Quantization along both axes and jagged
 * tensors" (square 32x32 blocks for Q, K and dO), with the scale rule of its
 * section "Softmax conversion and unroll-KV" (from the amax's exponent and
 * mantissa bits): the byte is that of the smallest power of two X with
 * amax / X <= 448 (X = 1 for an all-zero block); elements are divided by X
 * and rounded to the nearest e4m3 value (ties to even).
 *   x       device bf16, 16-byte aligned;  q: device bytes, 16-byte aligned
 *   scale   device bytes;  rows: multiple of 32;  d: 128
 * Errors: ATTN_E_HEADDIM, ATTN_E_SHAPE, ATTN_E_NULLPTR, ATTN_E_ALIGN, ATTN_E_HIP.
 */
int attn_mx_quantize(const void* x, uint8_t* q, uint8_t* scale, long long rows, int d, void* stream);

/*
 * attn_fwd_stats -- attn_fwd_ex that also counts lagging-max rescale events.
 *
 *   stats     device uint64 [4], accumulated into (the caller zeroes it):
 *             [0] row-block steps after a row's first block
 *             [1] of those, steps where the row committed a new max (a rescale)
 *             [2] 32-row group-block steps after the group's first block
 *             [3] of those, steps where any row of the group rescaled
 *             These are the "rows" and "warps" counts of the rescale-frequency
 *             table on "FlashAttention-4's Softmax Tricks". Counting adds
 *             atomics, so this entry point is for measurement, not speed.
 */
int attn_fwd_stats(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int Nq, int Nk, int d, int causal, float scale,
                   int exp2_mode, float tau, int dtype,
                   const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                   unsigned long long* stats, void* stream);

/*
 * attn_exp2 -- y[i] = 2^x[i] through the same device exp2 the attention kernels
 * inline (ATTN_EXP2_HW, ATTN_EXP2_EMU, ATTN_EXP2_EMU4 or ATTN_EXP2_EMU5; MIX is
 * not a per-element mode here).
 *   x, y      device float32 [n]; may alias
 *   n         >= 0
 * The software exp2 is defined for x <= 127 and returns 0 for x <= -127 and -inf.
 */
int attn_exp2(const float* x, float* y, long n, int exp2_mode, void* stream);

/* Emulated share used by ATTN_EXP2_MIX for (dtype, d, causal), in 16ths; < 0 on
 * an unsupported combination. */
int attn_mix_sixteenths(int dtype, int d, int causal);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
