// sage_prepass.hip -- smoothing and quantization pre-pass of libsage (gfx950).
//
// Implements, per (sequence, head):
//   * channel means (package page "sageattention", "What it is and what it
//     does": K smoothing; SageAttention2 summary, "Main concepts" item 2: Q
//     and V smoothing by channel-mean subtraction);
//   * INT8 codes with one FP32 scale per 64-token block for Q and K (package
//     page: per-block quantization of queries and keys; ComfyUI blog feature
//     item 2: Q.K^T in INT8); inside a whole forward call without Q
//     smoothing the fused kernel forms the Q codes itself, with the same
//     arithmetic, and this pass leaves Q out;
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
//           code = rne_e4m3(v_s*inv) (hardware convert, round to nearest even);
//   tiny a: where a < 2^-100 the quotients 127/a and 16256/a could leave
//           the FP32 range (a below about 10^-36, bf16 inputs), so the values
//           and a are scaled by 2^64 first (tiny_rescale: exact there, and the
//           codes are those of the block at any power-of-two scale); a V
//           channel that small counts as zero (scale 0, codes 0: the output
//           moves by less than 2^-100).
#include <type_traits>

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

__device__ inline float tiny_rescale(float a) { return a < 0x1p-100f ? 0x1p64f : 1.0f; }

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
// chunk's tokens, STAT_ABSMAX the max of |x - mu| (mu may be null).  A
// workgroup covers up to CPW consecutive 64-token chunks of one (sequence,
// head); thread (chunk j, granule e) owns channels 8e .. 8e+7 of chunk j and
// walks its tokens in order with 16-byte row reads.
// partial (s,h,g,c) at (((r_s/64)*heads + h*(np_s/64) + g)*d + c).
// ---------------------------------------------------------------------------
// One wave per statistics workgroup: its few chunks each still take one
// thread per granule walking the tokens in order, and the smaller
// workgroups give a small problem enough of them to cover the GPU (causal
// GQA, 16 MiB of K and V each: 512 rather than 128 of 256 threads).
constexpr int SWG = 64;

template <int D>
struct StatShape {
    static constexpr int GPR = D / 8;        // 16-byte granules per token row
    static constexpr int CPW = SWG / GPR;    // chunks per workgroup
};

// Workgroups sequence s owns in a statistics launch.
template <int D>
struct StatCount {
    const KParams* P;
    bool is_q;
    int heads;
    __device__ int operator()(int s) const {
        const int n = P->tab.uniform ? (is_q ? P->tab.nq[0] : P->tab.nkv[0])
                                     : (is_q ? P->tab.nq[s] : P->tab.nkv[s]);
        const int nch = (n + QBLK - 1) / QBLK;
        return heads * ((nch + StatShape<D>::CPW - 1) / StatShape<D>::CPW);
    }
};

template <int DT, int D, int MODE>
__device__ inline void stats_chunks(const KParams& P, const StatJob& J, int blk) {
    using SS = StatShape<D>;
    const bool is_q = J.which == 0;     // 0 = q, 1 = k, 2 = v
    int local;
    StatCount<D> cnt{&P, is_q, J.heads};
    const int s = find_seq(P, blk, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = is_q ? si.nq : si.nkv;
    const int nch = (n + QBLK - 1) / QBLK;
    const int ngrp = (nch + SS::CPW - 1) / SS::CPW;
    const int h = local / ngrp, grp = local % ngrp;
    const int j = threadIdx.x / SS::GPR, e = threadIdx.x % SS::GPR;
    const int g = grp * SS::CPW + j;                 // chunk of this thread
    if (j >= SS::CPW || g >= nch) return;
    const int64_t el0 = J.which == 0 ? si.q_el : (J.which == 1 ? si.k_el : si.v_el);
    const int64_t base = (is_q ? si.rq : si.rk) / QBLK * J.heads +
                         (int64_t)h * ((is_q ? si.npq : si.npk) / QBLK) + g;
    const uint16_t* x = J.x + el0 + (int64_t)h * J.xs.h + 8 * e;
    const int t0 = g * QBLK, t1 = min(t0 + QBLK, n);
    float m[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        m[k] = (MODE == STAT_ABSMAX && J.mu) ? J.mu[((int64_t)si.sid * J.heads + h) * D + 8 * e + k]
                                             : 0.0f;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) load8<DT>(x + (int64_t)(t + u) * J.xs.n, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if constexpr (MODE == STAT_SUM) acc[k] = acc[k] + v[u][k];
                else acc[k] = fmaxf(acc[k], fabsf(v[u][k] - m[k]));
            }
    }
    for (; t < t1; ++t) {
        float v[8];
        load8<DT>(x + (int64_t)t * J.xs.n, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (MODE == STAT_SUM) acc[k] = acc[k] + v[k];
            else acc[k] = fmaxf(acc[k], fabsf(v[k] - m[k]));
        }
    }
    float4* dst = reinterpret_cast<float4*>(J.partial + base * D + 8 * e);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

template <int DT, int D>
__device__ inline void stats_job_d(const KParams& P, const StatJob& J, int blk) {
    if (J.mode == STAT_SUM) stats_chunks<DT, D, STAT_SUM>(P, J, blk);
    else stats_chunks<DT, D, STAT_ABSMAX>(P, J, blk);
}

// Up to three statistics jobs in one launch; the grid is their block counts
// back to back.
template <int DT, int D>
__global__ __launch_bounds__(SWG) void k_stats(KParams P, StatJobs J) {
    int blk = blockIdx.x;
    if (blk < J.j[0].nblocks) { stats_job_d<DT, D>(P, J.j[0], blk); return; }
    blk -= J.j[0].nblocks;
    if (blk < J.j[1].nblocks) { stats_job_d<DT, D>(P, J.j[1], blk); return; }
    blk -= J.j[1].nblocks;
    stats_job_d<DT, D>(P, J.j[2], blk);
}

// ---------------------------------------------------------------------------
// Finalize per (sequence, head, channel).  STAT_SUM: mu = (chunk sums added in
// chunk order) / n.  STAT_ABSMAX: amax = max of the chunk maxima and
// scale = amax / 448 (0 below 2^-100).  A workgroup owns FIN_CH channels of one (sequence,
// head): it copies up to FIN_ROUND chunks of their partials into LDS with
// every load in flight at once, transposed so that each channel's values are
// contiguous, and thread c then combines channel c's values strictly in chunk
// order, four per LDS read.  Narrow channel slices keep the rounds few (one
// up to 28K tokens) and the workgroups many.
// ---------------------------------------------------------------------------
constexpr int FIN_ROUND = 448;              // chunks per LDS round (57 KB)

template <int MODE>
__device__ inline void finalize_one(const KParams& P, const FinJob& J, int blk, float* lds) {
    const int d = P.d;
    const int ns = d / FIN_CH;
    const int sh = blk / ns, slice = blk % ns;
    const int s = sh / J.heads, h = sh % J.heads;
    const int c = threadIdx.x;
    const SeqInfo si = seq_info(P, s);
    const int n = J.is_q ? si.nq : si.nkv;
    const int nch = (n + QBLK - 1) / QBLK;
    const int64_t base = (J.is_q ? si.rq : si.rk) / QBLK * J.heads +
                         (int64_t)h * ((J.is_q ? si.npq : si.npk) / QBLK);
    const float* src = J.partial + base * d + slice * FIN_CH;
    constexpr int G4 = FIN_CH / 4;          // float4 per chunk row of the slice
    constexpr int PER = FIN_ROUND * G4 / WG;
    float acc = 0.0f;
    for (int g0 = 0; g0 < nch; g0 += FIN_ROUND) {
        const int cnt = min(FIN_ROUND, nch - g0);
        float4 v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * WG;   // chunk idx / G4, float4 idx % G4
            if (idx < cnt * G4)
                v[i] = *reinterpret_cast<const float4*>(src + (int64_t)(g0 + idx / G4) * d +
                                                        4 * (idx % G4));
        }
        __syncthreads();                    // the previous round's sums are done
        // transposed image: channel row cc holds the round's chunks j at
        // lds[cc * (FIN_ROUND + 4) + j]
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * WG;
            if (idx < cnt * G4) {
                const int j = idx / G4, c4 = 4 * (idx % G4);
                lds[(c4 + 0) * (FIN_ROUND + 4) + j] = v[i].x;
                lds[(c4 + 1) * (FIN_ROUND + 4) + j] = v[i].y;
                lds[(c4 + 2) * (FIN_ROUND + 4) + j] = v[i].z;
                lds[(c4 + 3) * (FIN_ROUND + 4) + j] = v[i].w;
            }
        }
        __syncthreads();
        if (c < FIN_CH) {
            const float* row = lds + c * (FIN_ROUND + 4);
            int j = 0;
            for (; j + 16 <= cnt; j += 16) {
                float4 t[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) t[u] = *reinterpret_cast<const float4*>(row + j + 4 * u);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (MODE == STAT_SUM) acc = (((acc + t[u].x) + t[u].y) + t[u].z) + t[u].w;
                    else acc = fmaxf(fmaxf(fmaxf(fmaxf(acc, t[u].x), t[u].y), t[u].z), t[u].w);
                }
            }
            for (; j < cnt; ++j) {
                if constexpr (MODE == STAT_SUM) acc = acc + row[j];
                else acc = fmaxf(acc, row[j]);
            }
        }
    }
    if (c >= FIN_CH) return;
    const int64_t o = ((int64_t)si.sid * J.heads + h) * d + slice * FIN_CH + c;
    if constexpr (MODE == STAT_SUM) {
        J.out_mu[o] = n > 0 ? acc / (float)n : 0.0f;
    } else {
        J.out_amax[o] = acc;
        // a channel below 2^-100 counts as zero (its codes are 0 as well)
        J.out_scale[o] = acc >= 0x1p-100f ? acc / 448.0f : 0.0f;
    }
}

__device__ inline void finalize_job(const KParams& P, const FinJob& J, int blk, float* lds) {
    if (J.mode == STAT_SUM) finalize_one<STAT_SUM>(P, J, blk, lds);
    else finalize_one<STAT_ABSMAX>(P, J, blk, lds);
}

// Up to three finalize jobs (one workgroup per sequence, head and FIN_CH
// channels each).
__global__ __launch_bounds__(WG) void k_finalize(KParams P, FinJobs J) {
    __shared__ __align__(16) float lds[(FIN_ROUND + 4) * FIN_CH];
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
// QB: tokens per quantization block (64: the workgroup's whole chunk; 32:
// each half of it gets its own absmax and scale).
// With BQ (Q of a problem with per-block Q smoothing; `mu` is then NULL and
// `bq.mu_bar` the sequence mean), each quantization block is smoothed by its
// own channel mean (its valid tokens summed in order in FP32, divided by
// their count), and the block's deviation from the sequence mean,
// x = fl32(mu_b - mu_bar), is written as a 15-bit code: a = max |x|,
// inv = 16256/a, scale = a/16256, y = x*inv, hi = clamp(rne(y/128), +-127),
// lo = rne(y - 128*hi); blocks without a valid token get zeros.
struct BlockQ {
    const float* mu_bar;   // [S][hq][d]
    float* mu_b;           // per block [d]
    int8_t* code;          // per block [2][d]: hi, lo
    float* cscale;         // per block
};

template <int DT, int D, bool DELTA, int QB = QBLK, bool BQ = false>
__device__ inline void quant_qk_block(const KParams& P, const uint16_t* __restrict__ x,
                                      Strides xs, int is_q, int heads,
                                      const float* __restrict__ mu, int8_t* __restrict__ codes,
                                      float* __restrict__ scales,
                                      const float* __restrict__ mu_q,
                                      float* __restrict__ delta_s, int blkid, float* smf,
                                      BlockQ bq = BlockQ{}) {
    constexpr int GPR = D / 8;              // granules per token row
    constexpr int NG = QBLK * GPR;          // granules per block
    constexpr int PER = (NG + WG - 1) / WG; // granules per thread
    constexpr int NSUB = QBLK / QB;         // quantization blocks per chunk (1 or 2)
    float* red = smf;                       // NSUB * WG / 64 floats
    float* ks_lds = smf + 2 * (WG / 64);    // QBLK * D floats (DELTA, BQ)
    float* mub_lds = ks_lds + QBLK * D;     // NSUB * D floats (BQ)

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
    float amax[NSUB];
#pragma unroll
    for (int k = 0; k < NSUB; ++k) amax[k] = 0.0f;
    if constexpr (BQ) {
        // the chunk's raw values through LDS; thread c < NSUB*D sums channel
        // c % D of sub-block c / D down its valid tokens, in order
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int gi = threadIdx.x + i * WG;
            const int r = gi / GPR, cg = (gi % GPR) * 8;
            const int t = blk * QBLK + r;
#pragma unroll
            for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
            if (gi < NG && t < n) load8<DT>(x + el0 + (int64_t)t * xs.n + cg, val[i]);
            if (gi < NG) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ks_lds[r * D + cg + e] = val[i][e];
            }
        }
        __syncthreads();
        if (threadIdx.x < NSUB * D) {
            const int sub = threadIdx.x / D, ch = threadIdx.x % D;
            const int nvalid = min(QB, n - (blk * QBLK + sub * QB));
            float sum = 0.0f;
            for (int r = 0; r < nvalid; ++r) sum = sum + ks_lds[(sub * QB + r) * D + ch];
            const float m = nvalid > 0 ? sum / (float)nvalid : 0.0f;
            mub_lds[sub * D + ch] = m;
            bq.mu_b[(row0 / QB + blk * NSUB + sub) * D + ch] = m;
        }
        __syncthreads();
        // the deviation codes: wave `sub` codes sub-block sub
        const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (wv < NSUB) {
            const int nvalid = min(QB, n - (blk * QBLK + wv * QB));
            const float* mb = bq.mu_bar + ((int64_t)si.sid * heads + h) * D;
            float dv[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int c = lane + 64 * k;
                dv[k] = (c < D && nvalid > 0) ? mub_lds[wv * D + c] - mb[c] : 0.0f;
            }
            const float a = wave_max(fmaxf(fabsf(dv[0]), fabsf(dv[1])));
            const float rs = tiny_rescale(a);
            const float inv = a > 0.0f ? 16256.0f / (a * rs) : 0.0f;
            const int64_t ib = row0 / QB + blk * NSUB + wv;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int c = lane + 64 * k;
                if (c < D) {
                    const float y = (dv[k] * rs) * inv;
                    const float hi = fminf(fmaxf(rintf(y * 0.0078125f), -127.0f), 127.0f);
                    const float lo = rintf(y - 128.0f * hi);
                    bq.code[ib * 2 * D + c] = (int8_t)(int)hi;
                    bq.code[ib * 2 * D + D + c] = (int8_t)(int)lo;
                }
            }
            if (lane == 0) bq.cscale[ib] = a > 0.0f ? a / 16256.0f : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int gi = threadIdx.x + i * WG;
        const int r = gi / GPR, cg = (gi % GPR) * 8;
        const int t = blk * QBLK + r;
        if constexpr (!BQ) {
#pragma unroll
            for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
        }
        if (gi < NG && t < n) {
            if constexpr (BQ) {
                // (the raw values are already in registers)
                const float* mb = mub_lds + (NSUB == 1 || r < QB ? 0 : D);
#pragma unroll
                for (int e = 0; e < 8; ++e) val[i][e] = val[i][e] - mb[cg + e];
            } else {
                load8<DT>(x + el0 + (int64_t)t * xs.n + cg, val[i]);
                if (muh) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) val[i][e] = val[i][e] - muh[cg + e];
                }
            }
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(val[i][e]));
            if constexpr (NSUB == 1) amax[0] = fmaxf(amax[0], m);
            else if (r < QB) amax[0] = fmaxf(amax[0], m);
            else amax[1] = fmaxf(amax[1], m);
        }
    }
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
        const float wm = wave_max(amax[k]);
        if ((threadIdx.x & 63) == 0) red[k * (WG / 64) + (threadIdx.x >> 6)] = wm;
    }
    __syncthreads();
    float a[NSUB], inv[NSUB], rs[NSUB];
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
        a[k] = red[k * (WG / 64)];
#pragma unroll
        for (int w = 1; w < WG / 64; ++w) a[k] = fmaxf(a[k], red[k * (WG / 64) + w]);
        rs[k] = tiny_rescale(a[k]);
        inv[k] = a[k] > 0.0f ? 127.0f / (a[k] * rs[k]) : 0.0f;
    }
    // the codes; the rescale of tiny blocks (block-uniform) in a copy of its
    // own, so that other blocks run without it
    auto emit = [&](auto tiny) {
        constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int gi = threadIdx.x + i * WG;
            if (gi >= NG) continue;
            const int r = gi / GPR, cg = (gi % GPR) * 8;
            const bool first = NSUB == 1 || r < QB;
            const float inv_r = first ? inv[0] : inv[NSUB - 1];
            const float rs_r = first ? rs[0] : rs[NSUB - 1];
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = TINY ? val[i][e] * rs_r : val[i][e];
                float q = rintf(x * inv_r);
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
    };
    if (rs[0] != 1.0f || rs[NSUB - 1] != 1.0f) emit(std::true_type{});
    else emit(std::false_type{});
    if (threadIdx.x < NSUB) {
        const float av = threadIdx.x == 0 ? a[0] : a[NSUB - 1];
        scales[row0 / QB + blk * NSUB + threadIdx.x] = av > 0.0f ? av / 127.0f : 0.0f;
    }

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
// E4M3 quantization of one 128-token chunk of V (one key tile), written
// channel-major (V^T, so that the P.V operand of the fused kernel reads
// contiguous keys).  Codes pass through LDS for the transpose, and each
// channel's 128 codes leave as one whole 128-byte row segment (64-byte
// segments write measurably slower).  Tokens past the sequence end get zero
// codes.
// ---------------------------------------------------------------------------
constexpr int VQT = KVT;                     // tokens per E4M3 V chunk

template <int D>
constexpr int quant_v_lds_bytes() { return D * (VQT + 4); }

// Workgroups sequence s owns in the E4M3 V launch: heads x padded tiles.
struct VTileCount {
    const KParams* P;
    __device__ int operator()(int s) const {
        const int n = P->tab.uniform ? P->tab.nkv[0] : P->tab.nkv[s];
        return P->hkv * (round_up(n, KVT) / VQT);
    }
};

template <int DT, int D>
__device__ inline void quant_v_chunk(const KParams& P, const uint16_t* __restrict__ v,
                                     const float* __restrict__ mu,
                                     const float* __restrict__ amax,
                                     uint8_t* __restrict__ codes, int blkid, uint8_t* tr) {
    constexpr int GPR = D / 8;               // 8-channel granules of a token row
    constexpr int TASKS = GPR * (VQT / 4);   // (granule, group of 4 tokens) pairs
    constexpr int TS = VQT + 4;              // LDS bytes per channel row of the transpose

    int local;
    VTileCount cnt{&P};
    const int s = find_seq(P, blkid, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = si.nkv;
    const int nch = si.npk / VQT;
    const int h = local / nch, chk = local % nch;
    const int64_t el0 = si.v_el + (int64_t)h * P.vs.h;
    const float* muh = mu ? mu + ((int64_t)si.sid * P.hkv + h) * D : nullptr;
    const float* amh = amax + ((int64_t)si.sid * P.hkv + h) * D;

    // Each task reads 4 consecutive tokens of one granule (the granules of a
    // row are read by consecutive lanes) and leaves, per channel, the 4
    // codes as one 32-bit word of the channel's LDS row.  All of a thread's
    // row reads are issued before the first is converted.
    constexpr int NT = (TASKS + WG - 1) / WG;     // tasks per thread
    uint4 raw[NT][4];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int task = threadIdx.x + i * WG;
        const int cg = 8 * (task % GPR), tq = task / GPR;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = chk * VQT + 4 * tq + u;
            raw[i][u] = task < TASKS && t < n
                            ? *reinterpret_cast<const uint4*>(v + el0 + (int64_t)t * P.vs.n + cg)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int task = threadIdx.x + i * WG;
        if (task >= TASKS) break;
        const int cg = 8 * (task % GPR), tq = task / GPR;
        float inv[8], m8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = amh[cg + e];
            // below 2^-100 the channel counts as zero (its scale is 0 too)
            inv[e] = a >= 0x1p-100f ? 448.0f / a : 0.0f;
            m8[e] = muh ? muh[cg + e] : 0.0f;
        }
        uint32_t word[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) word[e] = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = chk * VQT + 4 * tq + u;
            if (t >= n) continue;                  // tokens past the end: zero codes
            const uint32_t w[4] = {raw[i][u].x, raw[i][u].y, raw[i][u].z, raw[i][u].w};
            float val[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                val[2 * k] = h2f<DT>((uint16_t)(w[k] & 0xffff));
                val[2 * k + 1] = h2f<DT>((uint16_t)(w[k] >> 16));
            }
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float x0 = muh ? val[e] - m8[e] : val[e];
                const float x1 = muh ? val[e + 1] - m8[e + 1] : val[e + 1];
                // a zero scale gives +0 codes (never the -0 of a negative x * 0)
                const float y0 = inv[e] > 0.0f ? x0 * inv[e] : 0.0f;
                const float y1 = inv[e + 1] > 0.0f ? x1 * inv[e + 1] : 0.0f;
                const uint32_t pk = e4m3_pk<false>(y0, y1, 0u);
                word[e] |= (pk & 0xffu) << (8 * u);
                word[e + 1] |= ((pk >> 8) & 0xffu) << (8 * u);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(tr + (cg + e) * TS + 4 * tq) = word[e];
    }
    __syncthreads();
    // store: channel c, 128 bytes = 8 x 16 B
    const int64_t vrow = (si.rk * P.hkv + (int64_t)h * si.npk) * D;
    for (int idx = threadIdx.x; idx < D * (VQT / 16); idx += WG) {
        const int c = idx / (VQT / 16), part = idx % (VQT / 16);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(tr + c * TS + part * 16);
        *reinterpret_cast<uint4*>(codes + vrow + (int64_t)c * si.npk + chk * VQT + part * 16) =
            make_uint4(src[0], src[1], src[2], src[3]);
    }
}

// The 16-bit V operand of the INT8-QK / 16-bit-PV variant (install guide
// "SageAttention量化加速框架", section 3.1: the qk_int8_pv_fp16 kernel): one
// 64-token chunk of one head, v (or v - mu_v, rounded to nearest even into
// the input's type) written channel-major like the E4M3 codes, 2 bytes per
// element.  Without smoothing the values are the input bits.
template <int DT>
__device__ inline uint32_t to16(float f) {
    if constexpr (DT == 0) {
        return (uint32_t)__half_as_ushort(__float2half_rn(f));
    } else {
        uint32_t u = __float_as_uint(f);
        u += 0x7fffu + ((u >> 16) & 1u);     // round to nearest even (inputs finite)
        return u >> 16;
    }
}

template <int D>
constexpr int half_v_lds_bytes() { return D * (2 * QBLK + 8); }

template <int DT, int D>
__device__ inline void half_v_chunk(const KParams& P, const uint16_t* __restrict__ v,
                                    const float* __restrict__ mu, uint16_t* __restrict__ out,
                                    int blkid, uint8_t* tr) {
    constexpr int GPR = D / 8;               // 8-channel granules of a token row
    constexpr int TASKS = GPR * (QBLK / 4);  // (granule, group of 4 tokens) pairs
    constexpr int TS = 2 * QBLK + 8;         // LDS bytes per channel row of the transpose

    int local;
    ChunkCount cnt{&P, false, P.hkv, 1};
    const int s = find_seq(P, blkid, cnt, &local);
    const SeqInfo si = seq_info(P, s);
    const int n = si.nkv;
    const int nch = si.npk / QBLK;
    const int h = local / nch, chk = local % nch;
    const int64_t el0 = si.v_el + (int64_t)h * P.vs.h;
    const float* muh = mu ? mu + ((int64_t)si.sid * P.hkv + h) * D : nullptr;

    // Each task reads 4 consecutive tokens of one granule and leaves, per
    // channel, the 4 values as 8 bytes of the channel's LDS row.
    for (int task = threadIdx.x; task < TASKS; task += WG) {
        const int cg = 8 * (task % GPR), tq = task / GPR;
        float m8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m8[e] = muh ? muh[cg + e] : 0.0f;
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = hi[e] = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = chk * QBLK + 4 * tq + u;
            if (t >= n) continue;                  // tokens past the end: zero
            float val[8];
            load8<DT>(v + el0 + (int64_t)t * P.vs.n + cg, val);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t b = to16<DT>(muh ? val[e] - m8[e] : val[e]);
                if (u < 2) lo[e] |= b << (16 * u);
                else hi[e] |= b << (16 * (u - 2));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint2*>(tr + (cg + e) * TS + 8 * tq) = make_uint2(lo[e], hi[e]);
    }
    __syncthreads();
    // store: channel c, 128 bytes = 8 x 16 B
    const int64_t vrow = (si.rk * P.hkv + (int64_t)h * si.npk) * D;
    for (int idx = threadIdx.x; idx < D * 8; idx += WG) {
        const int c = idx / 8, part = idx % 8;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(tr + c * TS + part * 16);
        *reinterpret_cast<uint4*>(out + vrow + (int64_t)c * si.npk + chk * QBLK + part * 8) =
            make_uint4(src[0], src[1], src[2], src[3]);
    }
}

// ---------------------------------------------------------------------------
// All quantization of a problem in one launch: the Q blocks, then the K
// blocks (with the score bias when Q is smoothed), then the V chunks.
// ---------------------------------------------------------------------------
template <int DT, int D, bool DELTA, int QB, bool BQ = false>
__global__ __launch_bounds__(WG) void k_quant(KParams P, QuantArgs A) {
    constexpr int QK_LDS = (2 * (WG / 64) + (DELTA || BQ ? QBLK * D : 0) + (BQ ? 2 * D : 0)) * 4;
    constexpr int VL = quant_v_lds_bytes<D>() > half_v_lds_bytes<D>() ? quant_v_lds_bytes<D>()
                                                                      : half_v_lds_bytes<D>();
    constexpr int LDS = QK_LDS > VL ? QK_LDS : VL;
    __shared__ __align__(16) uint8_t sm[LDS];
    int blk = blockIdx.x;
    if (blk < A.nq) {
        if constexpr (BQ)
            quant_qk_block<DT, D, false, QB, true>(
                P, A.q, P.qs, 1, P.hq, nullptr, A.q_codes, A.q_scale, nullptr, nullptr, blk,
                reinterpret_cast<float*>(sm), BlockQ{A.mu_q, A.mu_qb, A.mq_code, A.mq_scale});
        else
            quant_qk_block<DT, D, false, QB>(P, A.q, P.qs, 1, P.hq, A.mu_q, A.q_codes,
                                             A.q_scale, nullptr, nullptr, blk,
                                             reinterpret_cast<float*>(sm));
        return;
    }
    blk -= A.nq;
    if (blk < A.nk) {
        quant_qk_block<DT, D, DELTA, QB>(P, A.k, P.ks, 0, P.hkv, A.mu_k, A.k_codes, A.k_scale,
                                     A.mu_q, A.delta_s, blk, reinterpret_cast<float*>(sm));
        return;
    }
    blk -= A.nk;
    if (A.v_half)
        half_v_chunk<DT, D>(P, A.v, A.mu_v, reinterpret_cast<uint16_t*>(A.v_codes), blk, sm);
    else
        quant_v_chunk<DT, D>(P, A.v, A.mu_v, A.v_amax, A.v_codes, blk, sm);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int stat_chunks_per_wg(int d) { return SWG / (d / 8); }

hipError_t launch_stats(const KParams& P, int dtype, const StatJobs& J, hipStream_t st) {
    const int nb = J.j[0].nblocks + J.j[1].nblocks + J.j[2].nblocks;
    if (nb <= 0) return hipSuccess;
#define SAGE_ST(DT, D) k_stats<DT, D><<<nb, SWG, 0, st>>>(P, J)
    if (dtype == 0) {
        if (P.d == 64) SAGE_ST(0, 64); else if (P.d == 96) SAGE_ST(0, 96); else SAGE_ST(0, 128);
    } else {
        if (P.d == 64) SAGE_ST(1, 64); else if (P.d == 96) SAGE_ST(1, 96); else SAGE_ST(1, 128);
    }
#undef SAGE_ST
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
    if (P.qb == 32) {
        if (A.mq_code) k_quant<DT, D, true, 32, true><<<nb, WG, 0, st>>>(P, A);
        else if (A.delta_s) k_quant<DT, D, true, 32><<<nb, WG, 0, st>>>(P, A);
        else k_quant<DT, D, false, 32><<<nb, WG, 0, st>>>(P, A);
    } else {
        if (A.mq_code) k_quant<DT, D, true, QBLK, true><<<nb, WG, 0, st>>>(P, A);
        else if (A.delta_s) k_quant<DT, D, true, QBLK><<<nb, WG, 0, st>>>(P, A);
        else k_quant<DT, D, false, QBLK><<<nb, WG, 0, st>>>(P, A);
    }
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
