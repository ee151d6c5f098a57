// sage_internal.h -- shared host/device definitions of libsage (not part of
// the public ABI).  Kernel arguments are passed by value in `KParams`.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int QBLK = 64;      // Q/K quantization block (tokens)
constexpr int KVT = 128;      // key tile of the fused kernel (tokens)
constexpr int DEC_ROWS = 32;  // query rows of one wave of the decode kernel
constexpr int LDS_PER_CU = 160 * 1024;   // LDS bytes of one MI355X compute unit
constexpr int NUM_CU = 256;               // compute units of MI355X
constexpr int FIN_CH = 32;                // channels per statistics-finalize workgroup
constexpr int MAXSEQ = 32;    // sequences described per launch
constexpr int WG = 256;       // threads per workgroup of every kernel

struct Strides {
    int64_t b, h, n;          // elements; head_dim stride is 1
};

// Per-launch description of the sequences.  Dense problems use uniform = 1:
// every sequence has lengths nq[0], nkv[0], lives at batch index s and its
// padded row bases are s * npq and s * npk.  Variable-length problems list up
// to MAXSEQ sequences with token offsets into the packed tensors and their
// own padded row bases.
struct SeqTab {
    int32_t n;
    int32_t uniform;
    int32_t nq[MAXSEQ], nkv[MAXSEQ];
    int32_t tq[MAXSEQ], tk[MAXSEQ];     // first token (varlen)
    int64_t rq[MAXSEQ], rk[MAXSEQ];     // padded row bases in the code buffers
    int32_t sid[MAXSEQ];                // sequence index for [S][H][d] arrays and lse
    int64_t lse_base[MAXSEQ];           // first lse element of sequence s (head 0)
    int64_t dump0[MAXSEQ];              // first element of sequence s in the int32
                                        // Q.K^T test export (varlen)
};

struct KParams {
    int32_t d, hq, hkv, group;          // group = hq / hkv
    int32_t causal;
    int32_t pv_half;                    // P.V in the input's 16-bit type (else E4M3)
    int32_t qb;                         // tokens per Q/K quantization block (64 or 32)
    float sm_scale;                     // natural-log units
    float sml2;                         // sm_scale * log2(e)
    Strides qs, ks, vs, os;
    int64_t lse_hstride;                // elements between heads of lse
    // split key range (flash-decoding): kv_tiles key tiles per split (0: no
    // split), nsplit splits per sequence in the grid; each workgroup writes
    // its rows' partial (acc*v_scale + mu_v*l, m, l) at part_o / part_ml,
    // split-major over rows_total rows (the lse row index)
    int32_t kv_tiles, nsplit;
    int64_t rows_total;
    int32_t bqs;                        // per-block Q smoothing (bias formed in the kernel)
    // The fused kernel quantizes Q itself from this input tensor (null: it
    // reads the pre-pass codes); only where Q is not smoothed
    const uint16_t* q_raw;
    float* part_o;                      // [nsplit][rows_total][d]
    float* part_ml;                     // [nsplit][rows_total][2]: m (log2 units), l
    SeqTab tab;
};

// The merge of the split partials into the output (and lse).
struct MergeArgs {
    const float* part_o;
    const float* part_ml;
    int64_t rows_total;
    int32_t nsplit, d, hq, nq;          // nq: dense tokens per sequence
    int32_t varlen;
    int64_t total_q;                    // varlen: packed query tokens
    float poff;                         // log2 of the P scale folded into l (448 or 1)
    Strides os;
    void* o;
    float* lse;
};

struct SeqInfo {
    int nq, nkv, sid;
    int64_t q_el, k_el, v_el, o_el;     // element offset of (seq, head 0, token 0)
    int64_t rq, rk;                     // padded row bases
    int npq, npk;                       // padded lengths
    int64_t lse0;
};

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Two FP32 values converted to OCP E4M3 (round to nearest even) by the
// hardware's v_cvt_pk_fp8_f32 and written into the low (HI = false) or high
// 16 bits of `old`: every E4M3 code of the library (V codes, the P operand)
// and the test export of the conversion go through this one helper.
template <bool HI>
__device__ inline uint32_t e4m3_pk(float a, float b, uint32_t old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ inline SeqInfo seq_info(const KParams& P, int s) {
    const SeqTab& t = P.tab;
    SeqInfo r;
    if (t.uniform) {
        r.nq = t.nq[0];
        r.nkv = t.nkv[0];
        r.sid = s;
        r.q_el = (int64_t)s * P.qs.b;
        r.k_el = (int64_t)s * P.ks.b;
        r.v_el = (int64_t)s * P.vs.b;
        r.o_el = (int64_t)s * P.os.b;
        r.npq = round_up(r.nq, QBLK);
        r.npk = round_up(r.nkv, KVT);
        r.rq = (int64_t)s * r.npq;
        r.rk = (int64_t)s * r.npk;
        r.lse0 = (int64_t)s * P.hq * r.nq;
    } else {
        r.nq = t.nq[s];
        r.nkv = t.nkv[s];
        r.sid = t.sid[s];
        r.q_el = (int64_t)t.tq[s] * P.qs.n;
        r.k_el = (int64_t)t.tk[s] * P.ks.n;
        r.v_el = (int64_t)t.tk[s] * P.vs.n;
        r.o_el = (int64_t)t.tq[s] * P.os.n;
        r.npq = round_up(r.nq, QBLK);
        r.npk = round_up(r.nkv, KVT);
        r.rq = t.rq[s];
        r.rk = t.rk[s];
        r.lse0 = t.lse_base[s];
    }
    return r;
}

// Locate the sequence that owns linear block `blk` when sequence s owns
// `per(s)` consecutive blocks.  Returns the sequence and the local index.
template <typename F>
__device__ inline int find_seq(const KParams& P, int blk, F per, int* local) {
    if (P.tab.uniform) {
        int c = per(0);
        *local = blk % c;
        return blk / c;
    }
    int s = 0;
    for (; s < P.tab.n - 1; ++s) {
        int c = per(s);
        if (blk < c) break;
        blk -= c;
    }
    *local = blk;
    return s;
}

// Query heads of one GQA group that share a workgroup (1, 2 or 4); each wave
// owns 32 query rows of one of them.
__host__ __device__ inline int heads_per_wg(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

// ---- launchers (sage_prepass.hip, sage_attn.hip) ----
enum StatMode { STAT_SUM = 0, STAT_ABSMAX = 1 };

// One statistics job of the pre-pass: per-chunk channel sums (STAT_SUM) or
// absolute maxima of x - mu (STAT_ABSMAX) of one tensor (which: 0 q, 1 k, 2 v)
// into `partial`; nblocks = chunks x heads over the launch's sequences.
struct StatJob {
    const uint16_t* x;
    Strides xs;
    const float* mu;
    float* partial;
    int32_t which, heads, mode, nblocks;
};
struct StatJobs {
    StatJob j[3];   // unused entries have nblocks = 0
};
// One finalize job: per (sequence, head, channel) the mean (STAT_SUM, into
// out_mu) or the absolute maximum and its E4M3 scale (STAT_ABSMAX).
struct FinJob {
    const float* partial;
    float* out_mu;
    float* out_amax;
    float* out_scale;
    int32_t is_q, heads, mode, nblocks;
};
struct FinJobs {
    FinJob j[3];
};
// Everything the one-launch quantization needs.
struct QuantArgs {
    const uint16_t *q, *k, *v;
    const float *mu_q, *mu_k, *mu_v, *v_amax;
    int8_t *q_codes, *k_codes;
    uint8_t* v_codes;     // E4M3 codes, or 16-bit values when v_half
    float *q_scale, *k_scale, *delta_s;
    // per-block Q smoothing (mu_q is then the sequence mean): the block means,
    // the codes of their deviations from mu_q and the codes' scales
    float* mu_qb;
    int8_t* mq_code;
    float* mq_scale;
    int32_t nq, nk, nv;   // workgroups: Q blocks, K blocks, V chunks
    int32_t v_half;       // V operand kept 16-bit (no scale) instead of E4M3
};
// Chunks of 64 tokens one statistics workgroup covers (per sequence and head
// the launch needs ceil(chunks / this) workgroups).
int stat_chunks_per_wg(int d);
hipError_t launch_stats(const KParams& P, int dtype, const StatJobs& J, hipStream_t st);
hipError_t launch_finalize(const KParams& P, const FinJobs& J, hipStream_t st);
hipError_t launch_quant(const KParams& P, int dtype, const QuantArgs& A, hipStream_t st);
// mcode, mcs: the per-block Q smoothing codes and scales (P.bqs), else NULL.
hipError_t launch_attn(const KParams& P, int dtype, const int8_t* qc, const float* qsc,
                       const int8_t* kc, const float* ksc, const uint8_t* vc,
                       const float* vsc, const float* ds, const float* mu_v, void* o,
                       float* lse, const int8_t* mcode, const float* mcs, hipStream_t st);
// Workgroups of one fused-kernel launch before any key split.
int attn_base_wgs(const KParams& P);
// Whether a split launch runs the one-wave decode kernel: every sequence's
// GQA group times its queries fits the DEC_ROWS rows of one wave.
bool use_decode_kernel(const KParams& P);
// Waves of the decode kernel to place on one compute unit at once: at most
// one per SIMD (a fifth wave per unit, which the LDS would hold with FP8 V at
// d = 128, measured slower on the 32K-key decode workload), fewer when the
// LDS stages of a wave do not fit four times.
int decode_waves_per_cu(int d, bool pv_half, bool has_ds, int group);
hipError_t launch_merge(const MergeArgs& M, int dtype, hipStream_t st);
// The int32 Q.K^T of every (row, key) of the launch's sequences, written by
// the fused kernel's own staging and Q.K^T code (the test export; P.causal
// and the key split must be off, P.tab.dump0 set for varlen tables).
hipError_t launch_qk_dump(const KParams& P, const int8_t* qc, const int8_t* kc, int32_t* s_out,
                          hipStream_t st);
// The workspace of sage_attn_fwd_noalloc: the library's own static device
// array (NOALLOC_WS_MAX bytes, 256-byte aligned), one per device.  Returns
// its device address on the current device, taken once per device with
// hipGetSymbolAddress and kept.
constexpr size_t NOALLOC_WS_MAX = size_t{64} << 20;
hipError_t noalloc_workspace(void** ptr);

// E4M3 codes of the FP32 bit patterns first, first+1, ..., first+count-1,
// converted four per word as the fused kernel packs its P operand (the test
// export of the conversion).
hipError_t launch_e4m3_dump(uint32_t first, uint32_t count, uint8_t* out, hipStream_t st);

// Micro-benchmark rates (sage_micro.hip): the operation and its units per
// second, one timed launch over NUM_CU x 4 workgroups after a warm-up launch.
enum MicroOp { MICRO_I8 = 0, MICRO_F8 = 1, MICRO_EXP = 2, MICRO_FMA = 3 };
hipError_t micro_rate(int op, int reps, double* per_s, hipStream_t st);

}  // namespace sage
