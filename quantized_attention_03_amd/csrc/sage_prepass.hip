// sage_prepass.hip -- smoothing and quantization pre-pass of libsage (gfx950).
//
// Implements, per (sequence, head):
//   * channel means (package page "sageattention", "What it is and what it
//     does": K smoothing; SageAttention2 summary, "Main concepts" item 2: Q
//     and V smoothing by channel-mean subtraction);
//   * INT8 codes with one FP32 scale per 64-token block for Q and K (package
//     page: per-block quantization of queries and keys; ComfyUI blog feature
//     item 2: Q.K^T in INT8);
//   * OCP E4M3 codes with one FP32 scale per channel for V (ComfyUI blog
//     feature item 2: P.V in FP8, granularities differ);
//   * the score bias that compensates Q smoothing.
//
// All of it is HBM-bound elementwise work: lanes own channels or 16-byte
// granules of a token row, so every global access is a coalesced row read or
// write.  The arithmetic follows a fixed FP32 recipe (no contraction, fixed
// summation order, correctly rounded division, round-to-nearest-even) so that
// the results are reproducible bit for bit:
//   mean  : per 64-token chunk (aligned to the sequence start) sum the tokens
//           in order, then add the chunk sums in order, then one division;
//   int8  : a = max|x_s|, inv = 127/a, scale = a/127, code = rne(x_s*inv)
//           clamped to [-127, 127]; a == 0 -> scale 0, codes 0;
//   e4m3  : a = max over tokens |v_s|, inv = 448/a, scale = a/448,
//           code = rne_e4m3(v_s*inv) (hardware convert, round to nearest even).
#include "sage_internal.h"

#pragma clang fp contract(off)

namespace sage {

namespace {

template <int DT>
__device__ inline float h2f(uint16_t u) {
    if constexpr (DT == 0) {
        return __half2float(__ushort_as_half(u));
    } else {
        return __uint_as_float((uint32_t)u << 16);
    }
}

template <int DT>
__device__ inline void load8(const uint16_t* p, float* out) {
    uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = h2f<DT>((uint16_t)(w[i] & 0xffff));
        out[2 * i + 1] = h2f<DT>((uint16_t)(w[i] >> 16));
    }
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Number of blocks sequence s owns in a launch over (head, chunk) pairs.
struct ChunkCount {
    const KParams* P;
    bool is_q;
    int heads;
    int pad;   // 0: real chunks of 64 tokens; 1: padded length / 64
    __device__ int operator()(int s) const {
        int n = P->tab.uniform ? (is_q ? P->tab.nq[0] : P->tab.nkv[0])
                               : (is_q ? P->tab.nq[s] : P->tab.nkv[s]);
        int np = pad ? round_up(n, is_q ? QBLK : KVT) : round_up(n, QBLK);
        return heads * (np / QBLK);
    }
};

}  // namespace

// ---------------------------------------------------------------------------
// Per-chunk channel statistics: STAT_SUM gives the in-order FP32 sum of the
// chunk's tokens, STAT_ABSMAX the max of |x - mu| (mu may be null).  One
// workgroup per (sequence, head, 64-token chunk); thread c < d owns channel c
// and walks the chunk's tokens in order (each step is a coalesced row read).
// partial (s,h,g,c) at (((r_s/64)*heads + h*(np_s/64) + g)*d + c).
// ---------------------------------------------------------------------------
template <int DT, int MODE>
__device__ inline void stats_chunk(const KParams& P, const StatJob& J, int blk) {
    const bool is_q = J.which == 0;     // 0 = q, 1 = k, 2 = v
    int local;
    ChunkCount cnt{&P, is_q, J.heads, 0};
    const int s = find_seq(P, blk, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = is_q ? si.nq : si.nkv;
    const int nch = (n + QBLK - 1) / QBLK;
    const int h = local / nch, g = local % nch;
    const int d = P.d;
    const int64_t el0 = J.which == 0 ? si.q_el : (J.which == 1 ? si.k_el : si.v_el);
    const int64_t base = (is_q ? si.rq : si.rk) / QBLK * J.heads +
                         (int64_t)h * ((is_q ? si.npq : si.npk) / QBLK) + g;
    const int c = threadIdx.x;
    if (c >= d) return;
    const uint16_t* x = J.x;
    const int64_t off = el0 + (int64_t)h * J.xs.h + c;
    const int t0 = g * QBLK, t1 = min(t0 + QBLK, n);
    const float m = (MODE == STAT_ABSMAX && J.mu) ? J.mu[((int64_t)si.sid * J.heads + h) * d + c]
                                                  : 0.0f;
    float acc = 0.0f;
#pragma unroll 16
    for (int t = t0; t < t1; ++t) {
        const float v = h2f<DT>(x[off + (int64_t)t * J.xs.n]);
        if constexpr (MODE == STAT_SUM) {
            acc = acc + v;
        } else {
            acc = fmaxf(acc, fabsf(v - m));
        }
    }
    J.partial[base * d + c] = acc;
}

template <int DT>
__device__ inline void stats_job(const KParams& P, const StatJob& J, int blk) {
    if (J.mode == STAT_SUM) stats_chunk<DT, STAT_SUM>(P, J, blk);
    else stats_chunk<DT, STAT_ABSMAX>(P, J, blk);
}

// Up to three statistics jobs in one launch; the grid is their block counts
// back to back.
template <int DT>
__global__ __launch_bounds__(WG) void k_stats(KParams P, StatJobs J) {
    int blk = blockIdx.x;
    if (blk < J.j[0].nblocks) { stats_job<DT>(P, J.j[0], blk); return; }
    blk -= J.j[0].nblocks;
    if (blk < J.j[1].nblocks) { stats_job<DT>(P, J.j[1], blk); return; }
    blk -= J.j[1].nblocks;
    stats_job<DT>(P, J.j[2], blk);
}

// ---------------------------------------------------------------------------
// Finalize per (sequence, head, channel).  STAT_SUM: mu = (chunk sums added in
// chunk order) / n.  STAT_ABSMAX: amax = max of the chunk maxima and
// scale = amax / 448.  The workgroup first copies up to 64 chunks of partials
// into LDS (all loads in flight at once); thread c then combines its
// channel's values strictly in chunk order.
// ---------------------------------------------------------------------------
constexpr int FIN_CHUNKS = 64;

template <int MODE>
__device__ inline void finalize_one(const KParams& P, const FinJob& J, int blk, float* lds) {
    const int s = blk / J.heads, h = blk % J.heads;
    const int c = threadIdx.x;
    const int d = P.d;
    const SeqInfo si = seq_info(P, s);
    const int n = J.is_q ? si.nq : si.nkv;
    const int nch = (n + QBLK - 1) / QBLK;
    const int64_t base = (J.is_q ? si.rq : si.rk) / QBLK * J.heads +
                         (int64_t)h * ((J.is_q ? si.npq : si.npk) / QBLK);
    const float4* src = reinterpret_cast<const float4*>(J.partial + base * d);
    float acc = 0.0f;
    for (int g0 = 0; g0 < nch; g0 += FIN_CHUNKS) {
        const int cnt = min(FIN_CHUNKS, nch - g0);
        __syncthreads();
        for (int i = threadIdx.x; i < cnt * d / 4; i += WG) reinterpret_cast<float4*>(lds)[i] = src[g0 * d / 4 + i];
        __syncthreads();
        if (c < d) {
            for (int j = 0; j < cnt; ++j) {
                if constexpr (MODE == STAT_SUM) acc = acc + lds[j * d + c];
                else acc = fmaxf(acc, lds[j * d + c]);
            }
        }
    }
    if (c >= d) return;
    const int64_t o = ((int64_t)si.sid * J.heads + h) * d + c;
    if constexpr (MODE == STAT_SUM) {
        J.out_mu[o] = n > 0 ? acc / (float)n : 0.0f;
    } else {
        J.out_amax[o] = acc;
        J.out_scale[o] = acc / 448.0f;
    }
}

__device__ inline void finalize_job(const KParams& P, const FinJob& J, int blk, float* lds) {
    if (J.mode == STAT_SUM) finalize_one<STAT_SUM>(P, J, blk, lds);
    else finalize_one<STAT_ABSMAX>(P, J, blk, lds);
}

// Up to three finalize jobs (one workgroup per sequence and head each).
__global__ __launch_bounds__(WG) void k_finalize(KParams P, FinJobs J) {
    __shared__ __align__(16) float lds[FIN_CHUNKS * 128];
    int blk = blockIdx.x;
    if (blk < J.j[0].nblocks) { finalize_job(P, J.j[0], blk, lds); return; }
    blk -= J.j[0].nblocks;
    if (blk < J.j[1].nblocks) { finalize_job(P, J.j[1], blk, lds); return; }
    blk -= J.j[1].nblocks;
    finalize_job(P, J.j[2], blk, lds);
}

// ---------------------------------------------------------------------------
// INT8 quantization of one 64-token block of Q or K (padded blocks included:
// rows past the sequence end get zero codes; a block past the end gets scale
// 0).  256 threads; the block's 64 x d values are split in 16-byte granules
// of 8 channels; each thread keeps its granules' smoothed values in
// registers between the absmax reduction and the encode.
// With DELTA (K of a problem with Q smoothing), the block's smoothed rows are
// staged in LDS and ds[h_q][j] = sum_c mu_q[h_q][c] * k_s[j][c] (ascending c,
// FP32) is written for every query head of the group.
// ---------------------------------------------------------------------------
template <int DT, int D, bool DELTA>
__device__ inline void quant_qk_block(const KParams& P, const uint16_t* __restrict__ x,
                                      Strides xs, int is_q, int heads,
                                      const float* __restrict__ mu, int8_t* __restrict__ codes,
                                      float* __restrict__ scales,
                                      const float* __restrict__ mu_q,
                                      float* __restrict__ delta_s, int blkid, float* smf) {
    constexpr int GPR = D / 8;              // granules per token row
    constexpr int NG = QBLK * GPR;          // granules per block
    constexpr int PER = (NG + WG - 1) / WG; // granules per thread
    float* red = smf;                       // WG / 64 floats
    float* ks_lds = smf + WG / 64;          // QBLK * D floats (DELTA)

    int local;
    ChunkCount cnt{&P, is_q != 0, heads, 1};
    const int s = find_seq(P, blkid, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = is_q ? si.nq : si.nkv;
    const int np = is_q ? si.npq : si.npk;
    const int nblk = np / QBLK;
    const int h = local / nblk, blk = local % nblk;
    const int64_t el0 = (is_q ? si.q_el : si.k_el) + (int64_t)h * xs.h;
    const int64_t row0 = (is_q ? si.rq : si.rk) * heads + (int64_t)h * np;   // code row base
    const float* muh = mu ? mu + ((int64_t)si.sid * heads + h) * D : nullptr;

    float val[PER][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int gi = threadIdx.x + i * WG;
        const int r = gi / GPR, cg = (gi % GPR) * 8;
        const int t = blk * QBLK + r;
#pragma unroll
        for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
        if (gi < NG && t < n) {
            load8<DT>(x + el0 + (int64_t)t * xs.n + cg, val[i]);
            if (muh) {
#pragma unroll
                for (int e = 0; e < 8; ++e) val[i][e] = val[i][e] - muh[cg + e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(val[i][e]));
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    float a = red[0];
#pragma unroll
    for (int w = 1; w < WG / 64; ++w) a = fmaxf(a, red[w]);

    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int gi = threadIdx.x + i * WG;
        if (gi >= NG) continue;
        const int r = gi / GPR, cg = (gi % GPR) * 8;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = rintf(val[i][e] * inv);
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            const uint32_t b = (uint32_t)(int32_t)q & 0xffu;
            if (e < 4) w0 |= b << (8 * e); else w1 |= b << (8 * (e - 4));
        }
        *reinterpret_cast<uint2*>(codes + (row0 + blk * QBLK + r) * D + cg) = make_uint2(w0, w1);
        if constexpr (DELTA) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ks_lds[r * D + cg + e] = val[i][e];
        }
    }
    if (threadIdx.x == 0) scales[row0 / QBLK + blk] = a > 0.0f ? a / 127.0f : 0.0f;

    if constexpr (DELTA) {
        __syncthreads();
        // rows x query heads of the group; rows past the end get 0
        const int G = P.group;
        for (int idx = threadIdx.x; idx < QBLK * G; idx += WG) {
            const int r = idx % QBLK, hg = idx / QBLK;
            const int hq = h * G + hg;
            const int t = blk * QBLK + r;
            float acc = 0.0f;
            if (t < n) {
                const float* mq = mu_q + ((int64_t)si.sid * P.hq + hq) * D;
                for (int c = 0; c < D; ++c) acc = acc + mq[c] * ks_lds[r * D + c];
            }
            delta_s[si.rk * P.hq + (int64_t)hq * si.npk + t] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// E4M3 quantization of one 64-token chunk of V, written channel-major
// (V^T, so that the P.V operand of the fused kernel reads contiguous keys).
// Codes pass through LDS for the transpose; chunks past the sequence end and
// tokens past it get zero codes.
// ---------------------------------------------------------------------------
template <int D>
constexpr int quant_v_lds_bytes() { return D * (QBLK + 4); }

template <int DT, int D>
__device__ inline void quant_v_chunk(const KParams& P, const uint16_t* __restrict__ v,
                                     const float* __restrict__ mu,
                                     const float* __restrict__ amax,
                                     uint8_t* __restrict__ codes, int blkid, uint8_t* tr) {
    constexpr int GPR = D / 8;
    constexpr int NG = QBLK * GPR;
    constexpr int PER = (NG + WG - 1) / WG;
    constexpr int TS = QBLK + 4;            // LDS row stride (bytes) of the transpose

    int local;
    ChunkCount cnt{&P, false, P.hkv, 1};
    const int s = find_seq(P, blkid, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = si.nkv;
    const int nch = si.npk / QBLK;
    const int h = local / nch, chk = local % nch;
    const int64_t el0 = si.v_el + (int64_t)h * P.vs.h;
    const float* muh = mu ? mu + ((int64_t)si.sid * P.hkv + h) * D : nullptr;
    const float* amh = amax + ((int64_t)si.sid * P.hkv + h) * D;

#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int gi = threadIdx.x + i * WG;
        if (gi >= NG) continue;
        const int r = gi / GPR, cg = (gi % GPR) * 8;
        const int t = chk * QBLK + r;
        float val[8];
        uint8_t b[8];
        if (t < n) {
            load8<DT>(v + el0 + (int64_t)t * P.vs.n + cg, val);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                float x0 = muh ? val[e] - muh[cg + e] : val[e];
                float x1 = muh ? val[e + 1] - muh[cg + e + 1] : val[e + 1];
                const float a0 = amh[cg + e], a1 = amh[cg + e + 1];
                x0 = a0 > 0.0f ? x0 * (448.0f / a0) : 0.0f;
                x1 = a1 > 0.0f ? x1 * (448.0f / a1) : 0.0f;
                const uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0u, false);
                b[e] = (uint8_t)(pk & 0xff);
                b[e + 1] = (uint8_t)((pk >> 8) & 0xff);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = 0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tr[(cg + e) * TS + r] = b[e];
    }
    __syncthreads();
    // store: channel c, 64 bytes = 4 x 16 B
    const int64_t vrow = (si.rk * P.hkv + (int64_t)h * si.npk) * D;
    for (int idx = threadIdx.x; idx < D * 4; idx += WG) {
        const int c = idx / 4, part = idx % 4;
        const uint8_t* src = tr + c * TS + part * 16;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)src[4 * k] | ((uint32_t)src[4 * k + 1] << 8) |
                   ((uint32_t)src[4 * k + 2] << 16) | ((uint32_t)src[4 * k + 3] << 24);
        *reinterpret_cast<uint4*>(codes + vrow + (int64_t)c * si.npk + chk * QBLK + part * 16) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ---------------------------------------------------------------------------
// All quantization of a problem in one launch: the Q blocks, then the K
// blocks (with the score bias when Q is smoothed), then the V chunks.
// ---------------------------------------------------------------------------
template <int DT, int D, bool DELTA>
__global__ __launch_bounds__(WG) void k_quant(KParams P, QuantArgs A) {
    constexpr int QK_LDS = (WG / 64 + (DELTA ? QBLK * D : 0)) * 4;
    constexpr int LDS = QK_LDS > quant_v_lds_bytes<D>() ? QK_LDS : quant_v_lds_bytes<D>();
    __shared__ __align__(16) uint8_t sm[LDS];
    int blk = blockIdx.x;
    if (blk < A.nq) {
        quant_qk_block<DT, D, false>(P, A.q, P.qs, 1, P.hq, A.mu_q, A.q_codes, A.q_scale,
                                     nullptr, nullptr, blk, reinterpret_cast<float*>(sm));
        return;
    }
    blk -= A.nq;
    if (blk < A.nk) {
        quant_qk_block<DT, D, DELTA>(P, A.k, P.ks, 0, P.hkv, A.mu_k, A.k_codes, A.k_scale,
                                     A.mu_q, A.delta_s, blk, reinterpret_cast<float*>(sm));
        return;
    }
    blk -= A.nk;
    quant_v_chunk<DT, D>(P, A.v, A.mu_v, A.v_amax, A.v_codes, blk, sm);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_stats(const KParams& P, int dtype, const StatJobs& J, hipStream_t st) {
    const int nb = J.j[0].nblocks + J.j[1].nblocks + J.j[2].nblocks;
    if (nb <= 0) return hipSuccess;
    if (dtype == 0) k_stats<0><<<nb, WG, 0, st>>>(P, J);
    else k_stats<1><<<nb, WG, 0, st>>>(P, J);
    return hipGetLastError();
}

hipError_t launch_finalize(const KParams& P, const FinJobs& J, hipStream_t st) {
    const int nb = J.j[0].nblocks + J.j[1].nblocks + J.j[2].nblocks;
    if (nb <= 0) return hipSuccess;
    k_finalize<<<nb, WG, 0, st>>>(P, J);
    return hipGetLastError();
}

template <int DT, int D>
static void quant_d(const KParams& P, const QuantArgs& A, int nb, hipStream_t st) {
    if (A.delta_s) k_quant<DT, D, true><<<nb, WG, 0, st>>>(P, A);
    else k_quant<DT, D, false><<<nb, WG, 0, st>>>(P, A);
}

hipError_t launch_quant(const KParams& P, int dtype, const QuantArgs& A, hipStream_t st) {
    const int nb = A.nq + A.nk + A.nv;
    if (nb <= 0) return hipSuccess;
#define SAGE_QA(DT, D) quant_d<DT, D>(P, A, nb, st)
    if (dtype == 0) {
        if (P.d == 64) SAGE_QA(0, 64); else if (P.d == 96) SAGE_QA(0, 96); else SAGE_QA(0, 128);
    } else {
        if (P.d == 64) SAGE_QA(1, 64); else if (P.d == 96) SAGE_QA(1, 96); else SAGE_QA(1, 128);
    }
#undef SAGE_QA
    return hipGetLastError();
}

}  // namespace sage
