/*
 * sage.h -- C ABI of libsage: the SageAttention / SageAttention2 quantized
 * attention forward pass (INT8 Q.K^T, FP8 P.V) for AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed (cited by page title and section):
 *  - "sageattention" package page, "Quickstart": one call
 *    sageattn(q, k, v, tensor_layout, is_causal, smooth_k) returns the
 *    attention output; "What it is and what it does": K is smoothed, Q and K
 *    are quantized per block, head dim is 64, 96 or 128, Nq may differ from
 *    Nkv, GQA and variable sequence lengths are supported.
 *  - ComfyUI blog on SageAttention, feature list item 2: Q.K^T runs in INT8
 *    and P.V in FP8, with different quantization granularities; causal
 *    attention is supported (item 3).
 *  - "SageAttention2: technical report" summary, "Main concepts" item 2: Q
 *    and V may also be smoothed by subtracting their per-channel mean.
 *
 * The recipe, per (sequence, head):
 *   mu_x[c]   = mean over all tokens of the sequence of x[t][c] (x = q, k, v),
 *               FP32, chunks of 64 tokens summed in order, chunk sums added
 *               in order, one correctly rounded division by the length;
 *   x_s       = x - mu_x (FP32) when the smoothing flag of x is set, else x;
 *   Q, K      : per 64-token block (aligned to the sequence start), a = max|x_s|,
 *               scale = a/127, code = clamp(rne(x_s * (127/a)), -127, 127),
 *               a == 0 gives scale 0 and zero codes;
 *   V         : per channel over the sequence, a = max|v_s|, scale = a/448,
 *               code = e4m3(v_s * (448/a)) rounded to nearest even (OCP E4M3);
 *   ds[j]     = mu_q . k_s[j] (only with smooth_q; restores the scores that
 *               Q smoothing shifts by a key-dependent amount);
 *   s_ij      = (qc_i . kc_j) * sq * sk * sm_scale (+ ds[j] * sm_scale);
 *   online softmax over 128-key tiles with p^ = e4m3(448 * e^(s - m)),
 *   l summed from the FP32 p, o = sum p^ v^ * (v_scale/448) / l (+ mu_v).
 *
 * Finer Q/K blocks (qk_block = 32): the same INT8 quantization per 32-token
 * block, one wave's query rows and one 32-key MFMA block -- the gfx950 form
 * of SageAttention2's finer, thread-level quantization of Q and K
 * (SageAttention2 summary, "Main concepts"; package page: per-block
 * quantization).
 *
 * The 16-bit P.V variant (pv_mode = SAGE_PV_HALF), the first SageAttention's
 * INT8-QK / 16-bit-PV kernel (install guide "SageAttention量化加速框架",
 * section 3.1, the qk_int8_pv_fp16 benchmark; package page "What it is and
 * what it does": FP16 accumulators), changes only the P.V operands:
 *   V         : kept in the input's 16-bit type (v, or v - mu_v rounded to
 *               nearest even into that type), no scale;
 *   p^        = e^(s - m) rounded to nearest even into the same type,
 *   o = sum p^ v / l (+ mu_v), accumulated in FP32 (the MFMA's accumulator).
 *
 * A split key range (kv_split != 0; flash-decoding, for few queries against
 * long key ranges): the keys are cut into splits of kv_split keys, each split
 * runs the online softmax above from scratch, and the partial results are
 * merged by the log-sum-exp rule: M = max m_s, w_s = e^(m_s - M),
 * o = sum w_s acc_s / sum w_s l_s (+ mu_v).  Since p^ is rounded relative to
 * each split's own running maximum, the split is part of the recipe (the LSE
 * does not depend on it).
 *   Causal masking is aligned bottom-right: row i sees keys j <= i + Nkv - Nq;
 *   a row that sees no key gives o = 0 and lse = -inf.
 *
 * Conventions of every entry point
 *  - All tensor pointers are device pointers; descriptors, cu_seqlens and
 *    size outputs are host pointers.  Every pointer is borrowed: the library
 *    never allocates, frees or retains device memory, and never prints.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns before it completes.  Inputs must stay alive and unmodified and
 *    the workspace must not be reused until that work has completed.  Calls
 *    on different streams with different workspaces may run concurrently.
 *  - A call enqueues kernel launches only (no memset, copy, allocation or
 *    synchronization), so it may be captured into a HIP graph once the same
 *    kind of call has run eagerly (the first launch of a kernel sets its LDS
 *    limit with hipFuncSetAttribute).
 *  - Argument checks run first, on the host, in a fixed order; the first
 *    failure is returned and nothing is launched or written.  Inputs must be
 *    finite (not checked).  No exception crosses this ABI.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define SAGE_API __attribute__((visibility("default")))
#else
#define SAGE_API
#endif

/* Quantization block of Q and K (tokens) and key tile of the online softmax. */
#define SAGE_QK_BLOCK 64
#define SAGE_KV_TILE 128

typedef enum {
    SAGE_OK = 0,
    SAGE_ERR_NULL = 1,       /* a required pointer is NULL                      */
    SAGE_ERR_DTYPE = 2,      /* dtype is not SAGE_F16 / SAGE_BF16               */
    SAGE_ERR_LAYOUT = 3,     /* layout is not SAGE_HND / SAGE_NHD               */
    SAGE_ERR_HEAD_DIM = 4,   /* head_dim not in {64, 96, 128}                   */
    SAGE_ERR_SHAPE = 5,      /* a size is non-positive or too large             */
    SAGE_ERR_GQA = 6,        /* hq is not a multiple of hkv                      */
    SAGE_ERR_STRIDE = 7,     /* a stride is negative or not a multiple of 8     */
    SAGE_ERR_ALIGN = 8,      /* a pointer is not 16-byte aligned                */
    SAGE_ERR_WORKSPACE = 9,  /* workspace smaller than sage_workspace_size()    */
    SAGE_ERR_SEQLENS = 10,   /* cu_seqlens not monotone / not starting at 0     */
    SAGE_ERR_ARCH = 11,      /* current device is not gfx950                    */
    SAGE_ERR_HIP = 12,       /* a HIP runtime call or kernel launch failed      */
    SAGE_ERR_FLAGS = 13      /* a flag, pv_mode, kv_split or qk_block is invalid */
} sage_status;

typedef enum { SAGE_F16 = 0, SAGE_BF16 = 1 } sage_dtype;

/* Operands of P.V: E4M3 P^ and V^ (SageAttention2, the default) or P^ and V
 * in the input's 16-bit type (the first SageAttention's variant). */
typedef enum { SAGE_PV_FP8 = 0, SAGE_PV_HALF = 1 } sage_pv_mode;

/* kv_split value that lets the library choose the split.  tiles is the
 * longest key range in SAGE_KV_TILE units; a split has
 * max(4, ceil(tiles / want)) tiles, and none is made if that covers them.
 * - Decode shapes (hq / hkv times the longest query count at most 32): these
 *   run one wave per (sequence, kv head, split), and want = max(2,
 *   floor(256 * w / (sequences * hkv))), where w = 4 waves per compute unit
 *   (fewer when a wave's LDS stages do not fit four times in 160 KB: 3 for
 *   16-bit V at head_dim 128).
 * - Other shapes: no split while the unsplit grid has at least 256
 *   workgroups; otherwise want = ceil(512 / workgroups).
 * The choice depends on the problem only; sage_kv_split_size reports it. */
#define SAGE_KV_SPLIT_AUTO (-1)

/* HND = [batch, heads, tokens, head_dim]; NHD = [batch, tokens, heads, head_dim].
 * Variable-length inputs are packed over the sequences: NHD = [tokens, heads,
 * head_dim], HND = [heads, tokens, head_dim]. */
typedef enum { SAGE_HND = 0, SAGE_NHD = 1 } sage_layout;

/* smooth_q = SAGE_SMOOTH_Q_BLOCK: each Q quantization block is smoothed by
 * its own channel mean mu_b (SageAttention2 summary, "Main concepts" item 2:
 * Q is smoothed by subtracting its channel mean before quantization; here the
 * mean is taken per block).  The scores then owe mu_b.k_j: the sequence
 * mean's share mu_q.k_j is the score bias delta_s (as with smooth_q = 1), and
 * the block's deviation (mu_b - mu_q).k_j is formed inside the fused kernel
 * from a 15-bit code of the deviation and the INT8 key codes.  Requires
 * SAGE_PV_FP8 (SAGE_ERR_FLAGS otherwise); a split key range then always uses
 * the fused kernel (never the one-wave decode kernel). */
#define SAGE_SMOOTH_Q_BLOCK 2

/* Problem descriptor.  Strides are in elements for (batch, head, token); the
 * head_dim stride is 1.  A stride triple of all zeros means "contiguous in
 * `layout`" (the dense shapes above; for varlen calls the packed shapes, where
 * the batch stride is unused).  Output o has the dtype and layout of q. */
typedef struct {
    int32_t dtype;           /* sage_dtype of q, k, v and o                       */
    int32_t layout;          /* sage_layout of q, k, v and o                      */
    int32_t batch;           /* B (dense calls; varlen calls pass the count)     */
    int32_t hq, hkv;         /* query heads, key/value heads (hq % hkv == 0)     */
    int32_t nq, nkv;         /* tokens per sequence (dense) or max (varlen)      */
    int32_t head_dim;        /* 64, 96 or 128                                     */
    int64_t q_stride[3];
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    int32_t is_causal;       /* 0/1, bottom-right aligned                         */
    int32_t smooth_q;        /* 0/1 (SA2-style Q smoothing, with score bias), or
                                SAGE_SMOOTH_Q_BLOCK (one Q mean per quantization
                                block; FP8 P.V only)                             */
    int32_t smooth_k;        /* 0/1 (default 1)                                   */
    int32_t smooth_v;        /* 0/1 (SA2-style V smoothing, mean added back)     */
    float sm_scale;          /* <= 0 selects 1/sqrt(head_dim)                     */
    int32_t pv_mode;         /* sage_pv_mode (default SAGE_PV_FP8)                */
    int32_t kv_split;        /* keys per split of the key range: 0 none (default),
                                a positive multiple of SAGE_KV_TILE, or
                                SAGE_KV_SPLIT_AUTO                                */
    int32_t qk_block;        /* tokens per Q/K quantization block: 0 or 64
                                (default), or 32                                  */
} sage_attn_desc;

/* Fill `desc` for a dense, contiguous problem with the API defaults
 * (non-causal, smooth_k on, 1/sqrt(d)).  Never fails; checks happen later. */
SAGE_API void sage_desc_init(sage_attn_desc* desc, int32_t dtype, int32_t layout, int32_t batch,
                    int32_t hq, int32_t hkv, int32_t nq, int32_t nkv, int32_t head_dim);

/*
 * Quantized tensors written by sage_quant_qkv (device memory, caller-owned).
 * Sequences are s = 0..S-1 (S = batch for dense calls).  Per sequence,
 * npq_s = nq_s rounded up to SAGE_QK_BLOCK and npk_s = nkv_s rounded up to
 * SAGE_KV_TILE; row bases rq_s = sum_{s'<s} npq_s' and rk_s = sum npk_s'.
 *   mu_q    [S][hq][d]  FP32, only if smooth_q (the sequence mean; may be
 *           NULL otherwise)
 *   mu_k    [S][hkv][d] FP32, only if smooth_k
 *   mu_v    [S][hkv][d] FP32, only if smooth_v
 *   q_codes int8: element (s,h,n,c) at ((rq_s*hq + h*npq_s + n)*d + c);
 *           rows n >= nq_s are zero
 *   q_scale FP32: (s,h,blk) at (rq_s*hq + h*npq_s)/QB + blk, QB = the
 *           descriptor's qk_block (64 unless 32 is asked for)
 *   k_codes int8: (s,h,n,c) at ((rk_s*hkv + h*npk_s + n)*d + c), pad rows zero
 *   k_scale FP32: (s,h,blk) at (rk_s*hkv + h*npk_s)/QB + blk (pad blocks 0)
 *   v_codes OCP E4M3 bytes, channel-major: (s,h,n,c) at
 *           ((rk_s*hkv + h*npk_s)*d + c*npk_s + n), pad tokens zero;
 *           with SAGE_PV_HALF the same index counts 16-bit elements of the
 *           input's type (v, or v - mu_v rounded into that type)
 *   v_scale FP32 [S][hkv][d] (unused with SAGE_PV_HALF: size 0, may be NULL)
 *   delta_s FP32: (s,h,n) at rk_s*hq + h*npk_s + n, only if smooth_q
 * With smooth_q = SAGE_SMOOTH_Q_BLOCK also, per (s,h,blk) at index
 * ib = (rq_s*hq + h*npq_s)/QB + blk (the index of q_scale; blocks without a
 * valid token hold zeros):
 *   mu_qb       FP32 [ib][d]: the block's channel mean (its valid tokens
 *               summed in order in FP32, divided by their count); q_codes
 *               are then of q - mu_qb
 *   mu_q_code   int8 [ib][2][d]: hi, lo of x = fl32(mu_qb - mu_q): with
 *               a = max |x|, y = x * fl32(16256/a), hi = clamp(rne(y/128),
 *               +-127), lo = rne(y - 128*hi)
 *   mu_q_cscale FP32 [ib]: fl32(a/16256) (0 when a = 0)
 * All pointers 16-byte aligned.
 */
typedef struct {
    float* mu_q;
    float* mu_k;
    float* mu_v;
    int8_t* q_codes;
    float* q_scale;
    int8_t* k_codes;
    float* k_scale;
    uint8_t* v_codes;
    float* v_scale;
    float* delta_s;
    float* mu_qb;
    int8_t* mu_q_code;
    float* mu_q_cscale;
} sage_quant_bufs;

/* Byte sizes of each sage_quant_bufs member for a problem (0 when unused). */
typedef struct {
    size_t mu_q, mu_k, mu_v, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, delta_s;
    size_t mu_qb, mu_q_code, mu_q_cscale;
} sage_quant_sizes;

/* Sizes for a dense call (cu_seqlens_* NULL, nseq ignored) or a varlen call
 * (host cu_seqlens_q / cu_seqlens_kv with nseq + 1 entries).  Returns the
 * same validation errors as the compute entry points. */
SAGE_API sage_status sage_quant_buf_sizes(const sage_attn_desc* desc, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv, int32_t nseq,
                                 sage_quant_sizes* sizes);

/* Device workspace bytes needed by sage_attn_fwd (varlen = 0) or
 * sage_attn_fwd_varlen (varlen = 1, cu_seqlens given); sage_quant_qkv and
 * sage_attn_fwd_quantized need at most the same. */
SAGE_API sage_status sage_workspace_size(const sage_attn_desc* desc, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_kv, int32_t nseq, size_t* bytes);

/*
 * sage_quant_qkv -- the pre-pass alone: channel means, smoothing, INT8 Q/K
 * per-block codes and scales, E4M3 V codes and per-channel scales (or the
 * 16-bit V operand with SAGE_PV_HALF), and the Q-smoothing score bias,
 * written to `out` in the layout above.  Dense when
 * cu_seqlens_q == NULL; otherwise varlen with host cu_seqlens_q/kv
 * (nseq + 1 int32 prefix offsets starting at 0, non-decreasing) and packed
 * q/k/v.  Sources: package page "What it is and what it does" (smoothing,
 * per-block quantization); ComfyUI blog feature item 2 (INT8 / FP8,
 * granularities); SageAttention2 summary "Main concepts" item 2 (Q, V
 * smoothing).  Bit-exact by construction with the FP32 recipe above.
 */
SAGE_API sage_status sage_quant_qkv(const sage_attn_desc* desc, const void* q, const void* k,
                           const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_kv, int32_t nseq,
                           const sage_quant_bufs* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * sage_attn_fwd -- full forward pass for dense inputs: pre-pass, then the
 * fused INT8-QK / online-softmax / FP8-PV (or 16-bit-PV) kernel.  q [B,hq,nq,d] (HND) or
 * [B,nq,hq,d] (NHD) with the descriptor's strides; k, v likewise with hkv,
 * nkv; o has q's shape.  lse (nullable) receives FP32 [B][hq][nq], the natural
 * log of sum_j e^(s_ij) over the scores as formed above (after smoothing).
 * The workspace holds the quantized tensors and partial sums.  Source:
 * package page "Quickstart" (the sageattn call this mirrors).
 */
SAGE_API sage_status sage_attn_fwd(const sage_attn_desc* desc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd_varlen -- the same for `nseq` packed sequences of different
 * lengths (package page, "What it is and what it does": variable sequence
 * lengths, Nq != Nkv).  cu_seqlens_q / cu_seqlens_kv are HOST arrays of
 * nseq + 1 int32 offsets (0 first, non-decreasing); sequence s owns query
 * tokens [cu_q[s], cu_q[s+1]) and key tokens [cu_kv[s], cu_kv[s+1]).  Each
 * sequence gets its own means, its own 64-token blocks aligned to its start,
 * and bottom-right causal alignment.  lse is FP32 [hq][total_q].
 */
SAGE_API sage_status sage_attn_fwd_varlen(const sage_attn_desc* desc, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv, int32_t nseq, const void* q,
                                 const void* k, const void* v, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd_noalloc -- sage_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments and checks as
 * sage_attn_fwd without the workspace: the workspace is the library's own
 * static device array of SAGE_NOALLOC_WS_MAX bytes, one per device, held
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  Problems whose workspace
 * (sage_workspace_size) exceeds SAGE_NOALLOC_WS_MAX return
 * SAGE_ERR_WORKSPACE.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it has to start at zero):
 * calls that overlap on one GPU (different streams, or host threads) race
 * and must be serialized by the caller.
 */
#define SAGE_NOALLOC_WS_MAX ((size_t)64 << 20)
SAGE_API sage_status sage_attn_fwd_noalloc(const sage_attn_desc* desc, const void* q,
                                           const void* k, const void* v, void* o, float* lse,
                                           void* stream);

/*
 * sage_attn_fwd_quantized -- the fused kernel alone, on tensors that
 * sage_quant_qkv wrote for the same descriptor and cu_seqlens (dense when
 * cu_seqlens_q == NULL).  Lets a caller quantize K/V once and attend to them
 * many times, and isolates the O(N^2) part for timing (SA1 abstract,
 * llama.cpp discussion #9901: this is where attention spends its time).
 * o and lse as in sage_attn_fwd / sage_attn_fwd_varlen.  The workspace holds
 * the split partials and is only used with a split key range (it may then
 * be any size from sage_workspace_size; otherwise NULL and 0 are accepted).
 */
SAGE_API sage_status sage_attn_fwd_quantized(const sage_attn_desc* desc,
                                             const int32_t* cu_seqlens_q,
                                             const int32_t* cu_seqlens_kv, int32_t nseq,
                                             const sage_quant_bufs* bufs, void* o, float* lse,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * sage_kv_split_size -- the keys per split the library uses for a problem
 * (0: no split): the descriptor's kv_split, or the SAGE_KV_SPLIT_AUTO
 * choice.  Same validation as the compute entry points.  Source: the
 * llama.cpp discussion #9901 (SA1 abstract) puts attention's cost in long
 * sequences; the split lets few queries use the whole GPU.
 */
SAGE_API sage_status sage_kv_split_size(const sage_attn_desc* desc, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_kv, int32_t nseq,
                                        int32_t* keys_per_split);

/*
 * sage_debug_qk_int32 -- test hook: the exact int32 Q^.K^^T of the codes in
 * `bufs` (as written by sage_quant_qkv for the same desc), computed by the
 * same device code as the fused kernel's Q.K^T stage.  s_out is device
 * int32 [S][hq][nq_s][nkv_s] packed over sequences (dense: [B][hq][nq][nkv]).
 * Source: ComfyUI blog feature item 2 (Q.K^T in INT8).
 */
SAGE_API sage_status sage_debug_qk_int32(const sage_attn_desc* desc, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_kv, int32_t nseq,
                                const sage_quant_bufs* bufs, int32_t* s_out, void* stream);

/*
 * sage_debug_e4m3_encode -- test hook: the OCP E4M3 codes of the FP32 values
 * whose bit patterns are first, first+1, ..., first+count-1 (first + count <=
 * 2^32), converted by the same device helper and in the same packing as every
 * E4M3 code of the library (the V codes of the pre-pass and the P operand of
 * the fused kernel), so that the conversion can be compared exhaustively with
 * a reference encoder.  out: device, count bytes, 16-byte aligned.  Errors:
 * SAGE_ERR_NULL (out NULL with count > 0), SAGE_ERR_ALIGN, SAGE_ERR_SHAPE
 * (the range passes 2^32), SAGE_ERR_ARCH, SAGE_ERR_HIP.  Source: ComfyUI blog
 * feature item 2 (P.V in FP8).
 */
SAGE_API sage_status sage_debug_e4m3_encode(uint32_t first, uint32_t count, uint8_t* out,
                                            void* stream);

/*
 * sage_micro_rate -- measured throughput of one execution unit the fused
 * kernel depends on, to set beside the part's published peak: the dense INT8
 * matrix instruction of Q.K^T (v_mfma_i32_32x32x32_i8) and the FP8 one of P.V
 * (v_mfma_scale_f32_32x32x64_f8f6f4), in operations (2 per multiply-add) per
 * second; v_exp_f32 in results per second; v_fma_f32 in flops per second.
 * One launch of independent dependency chains over 4 workgroups of 512
 * threads per compute unit, `reps` iterations each (1 .. 2^20; 4096 takes
 * about 2 ms for the matrix operations), timed with events on `stream` after
 * a warm-up launch.  Blocks until the launches end.  Errors: SAGE_ERR_NULL
 * (rate), SAGE_ERR_FLAGS (op), SAGE_ERR_SHAPE (reps), SAGE_ERR_ARCH,
 * SAGE_ERR_HIP.  Source: ComfyUI blog feature item 2 (INT8 Q.K^T, FP8 P.V).
 */
typedef enum { SAGE_MICRO_I8 = 0, SAGE_MICRO_F8 = 1, SAGE_MICRO_EXP = 2, SAGE_MICRO_FMA = 3 } sage_micro_op;
SAGE_API sage_status sage_micro_rate(int32_t op, int32_t reps, double* rate, void* stream);

/* Human-readable name of a status code (static storage); any other value
 * gives "unknown status".  (The code is taken as an integer, so that a value
 * outside the enumeration is well defined.) */
SAGE_API const char* sage_status_string(int32_t status);

/* SAGE_ABI_VERSION of the built library. */
SAGE_API int32_t sage_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H */
