// sage_attn.hip -- fused quantized attention forward for gfx950 (CDNA4).
//
// What it computes (ComfyUI blog on SageAttention, feature item 2: Q.K^T in
// INT8, P.V in FP8; SA1 abstract in llama.cpp discussion #9901: the O(N^2)
// part of attention is the one quantized; FlashAttention-style tiling with an
// online softmax), per query row i of one (sequence, query head):
//   s_ij = (qc_i . kc_j) * sq_i * sk_j * sm_scale (+ ds_j * sm_scale)
//   online softmax over 128-key tiles, p^ = e4m3(448 * 2^(s*log2e - m)),
//   l accumulated from the FP32 p, o_i = sum p^ v^ * (v_scale / 448) / l (+ mu_v).
// ds_j compensates Q smoothing: mu_q . k_j for one mean per sequence, plus,
// with one mean per Q block, the block's deviation from it, formed here from
// its code and the INT8 key codes (see Bqs below).
//
// Design for CDNA4:
//  * A wave owns 32 query rows of one query head.  With GQA, the waves of a
//    workgroup take up to 4 query heads of one key/value head so that every
//    K/V tile staged in LDS feeds all of them.
//  * S^T = Kc . Qc^T on v_mfma_i32_32x32x32_i8 (A = key rows from LDS,
//    B = the wave's Q codes held in VGPRs).  The accumulators start at the
//    bits of 1.5*2^23, so each score S is recovered exactly as a float by one
//    subtraction; the row max is a float max tree over the exact S of each
//    block of keys that shares a scale, scaled once per block, and each score
//    then costs one FMA, x = S * (sq*sk*sm_scale*log2 e) - (m - log2 448),
//    rounded once.
//  * Key rows are fed to the MFMA in a permuted order so that in the output
//    layout each lane holds 16 consecutive keys of its own query row; lanes l
//    and l+32 share a row, so the row max needs a single permlane32 swap.
//  * O^T += V^T . P^T on v_mfma_f32_32x32x64_f8f6f4: the P operand is exactly
//    the lane's own scores converted pairwise with v_cvt_pk_fp8_f32 (no
//    relayout); V^T comes from LDS as two 16-byte reads per lane.  The
//    accumulator layout keeps each lane on its own query row, so the
//    rescale by alpha and the final 1/l need no cross-lane traffic.
//  * K and V^T tiles are double-buffered in LDS and filled by direct global ->
//    LDS loads (no staging registers); 16-byte slots of each LDS row are
//    XOR-swizzled so the operand reads are bank-conflict free.
//  * Ping-pong: a workgroup has 8 waves in two groups of 4; the two waves
//    that share a SIMD belong to different groups.  Each group alternates an
//    MFMA phase and a softmax phase, offset by one phase from the other
//    group, with a workgroup barrier between phases.  The MFMA phase holds
//    the alpha rescale of O and the P.V of tile t-1, then Q.K(t)^T, at
//    raised priority; the softmax phase the score half of tile t (exact S,
//    row max, exponent FMA, v_exp_f32) and its operand half (the row sum of
//    p and the FP8 packing).  At d = 64, where the softmax phase is the whole
//    bound, the operand half moves to the next MFMA phase, under its matrix
//    instructions (a single wave issues VALU work only about every fifth
//    cycle, about half of what the SIMD takes from two waves).
//  * Causal (bottom-right) masking and sequence tails are applied only on
//    the tiles that straddle them; fully hidden tiles are skipped.
//  * Inside a whole forward call without Q smoothing the kernel quantizes its
//    own Q rows in its prologue (the pre-pass then skips Q); otherwise, and
//    in the entry point that takes caller codes, it reads the Q codes
//    (q_load / q_values / q_codes).
//  * Row maxima beyond 2^16 in log2 units are raised a few units in their
//    last place (raise_max), so that no P code reaches the E4M3 NaN code.
#include <algorithm>
#include <atomic>
#include <cfloat>
#include <mutex>
#include <vector>

#include "sage_internal.h"

namespace sage {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float LOG2_448 = 8.807354922057604f;
constexpr int SBIAS_I = 0x4B400000;
constexpr float SBIAS_F = 12582912.0f;
constexpr int NEG_INF_BITS = (int)0xFF800000u;   // -inf as a float, negative as an integer
constexpr float LN2 = 0.6931471805599453f;
constexpr int FWD_WAVES = 8;               // waves per workgroup of the fused kernel
constexpr int FWD_NT = 64 * FWD_WAVES;

template <int D, bool PVH = false>
struct Tile {
    // LDS image of one 128-key tile.  K rows are 128 bytes (64 for D = 64;
    // D = 96 leaves two 16-byte slots of a row unused); V^T rows (one per
    // channel) are 128 bytes, and the V^T stage is padded to 128 rows for
    // D = 96 so that it is a whole number of 8 KB copies.  Rows are dense and
    // their 16-byte slots are XOR-swizzled (slot = granule ^ swz(row)) so that
    // the MFMA operand reads of 16 consecutive rows hit distinct banks.
    // With 16-bit P.V operands (PVH) a V^T row holds 128 two-byte values.
    static constexpr int KRS = D == 64 ? 64 : 128;
    static constexpr int KBYTES = KVT * KRS;
    static constexpr int VROWS = D == 96 ? 128 : D;
    static constexpr int VES = PVH ? 2 : 1;           // bytes per V element
    static constexpr int VRB = KVT * VES;             // bytes per V^T row
    static constexpr int VBYTES = VROWS * VRB;
    static constexpr int DSBYTES = 4 * KVT * 4;  // score bias, per head of the workgroup
};

template <int RS>
__device__ inline int swz(int row) {
    if constexpr (RS == 256) return row & 15;
    else if constexpr (RS == 128) return (row & 7) ^ ((row >> 3) & 1);
    else return ((row >> 1) & 3) ^ ((row >> 3) & 1);
}

// Key held by LDS row r of a tile: within each 32-row block, row i holds key
// 16*((i/4)%2) + 4*(i/8) + i%4, so that the S^T output register r of lane
// (row, half) is key 32b + 16*half + r.
__device__ inline int key_of_row(int r) {
    const int i = r & 31;
    return (r & ~31) + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ inline void dma16(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds_wave_base, 16, 0, 0);
}

// Wait for this wave's outstanding memory operations (the direct-to-LDS
// copies included), then the workgroup barrier.
__device__ inline void bar() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Per-lane source offsets of the global -> LDS tile copies of a workgroup of
// NT threads.  Copy i moves NT*16 bytes: lane L of wave w writes
// base + NT*16*i + 1024*w + 16*L, and its source is chosen so that the
// swizzled LDS image results.  The key permutation and the swizzle repeat
// every 32 rows and a copy spans a multiple of 32 rows, so copy i's source is
// copy 0's plus a constant: one offset per tensor suffices.
template <int D, int NT, bool PVH = false>
struct DmaOffsets {
    using TT = Tile<D, PVH>;
    static constexpr int KCOPIES = TT::KBYTES / (NT * 16);
    static constexpr int VCOPIES = TT::VBYTES / (NT * 16);
    static constexpr int KROWS = NT * 16 / TT::KRS;        // key rows per copy
    static constexpr int VROWS = NT * 16 / TT::VRB;        // V^T rows per copy
    static_assert(KCOPIES * NT * 16 == TT::KBYTES && KROWS % 32 == 0, "K copy shape");
    static_assert(VCOPIES * NT * 16 == TT::VBYTES && VROWS % 16 == 0, "V copy shape");
    int k0;   // bytes from the key tile start (row-major codes)
    int v0;   // bytes from the V^T tile start (channel rows of npk elements)

    __device__ inline void init(int npk) {
        using T = TT;
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
        const int o = w * 1024 + lane * 16;
        const int row = o / T::KRS, slot = (o % T::KRS) / 16;
        int lg = slot ^ swz<T::KRS>(row);
        if (D == 96 && lg >= 6) lg &= 1;           // unused slots: any in-row granule
        k0 = key_of_row(row) * D + lg * 16;
        const int ch = o / T::VRB, vslot = (o % T::VRB) / 16;
        v0 = ch * npk * T::VES + ((vslot ^ swz<T::VRB>(ch)) << 4);
    }
};

// Issue this thread's copies of K tile t (and of the per-head score bias of
// the tile, which has its own stage) into LDS.
template <int D, int NT, bool HAS_DS, bool PVH = false>
__device__ inline void stage_k(uint8_t* kst, uint8_t* dsst, const DmaOffsets<D, NT, PVH>& off,
                               const int8_t* kbase, const float* dsb, int npk, int t, int hpw) {
    using O = DmaOffsets<D, NT, PVH>;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int8_t* kt = kbase + (int64_t)t * KVT * D;
#pragma unroll
    for (int i = 0; i < O::KCOPIES; ++i)
        dma16(kt + off.k0 + i * O::KROWS * D, kst + i * NT * 16 + w * 1024);
    if constexpr (HAS_DS) {
        // hpw heads x 128 floats; waves 0 and 1 cover up to 4 heads
        if (w * 2 < hpw) {
            int hs = w * 2 + lane / 32;
            if (hs >= hpw) hs = hpw - 1;
            dma16(dsb + (int64_t)hs * npk + t * KVT + (lane % 32) * 4, dsst + w * 1024);
        }
    }
}

// Issue this thread's copies of V^T tile t into LDS.
template <int D, int NT, bool PVH = false>
__device__ inline void stage_v(uint8_t* vst, const DmaOffsets<D, NT, PVH>& off,
                               const uint8_t* vbase, int npk, int t) {
    using O = DmaOffsets<D, NT, PVH>;
    using T = Tile<D, PVH>;
    const int w = threadIdx.x >> 6;
    const uint8_t* vt = vbase + t * (KVT * T::VES);
#pragma unroll
    for (int i = 0; i < O::VCOPIES; ++i) {
        // D = 96: rows 96..127 of the stage are padding; their copies read
        // channels 0..31 again (any valid source)
        const int dst_ch = i * O::VROWS + (threadIdx.x * 16) / T::VRB;
        const int64_t rows = (int64_t)i * O::VROWS - ((D == 96 && dst_ch >= 96) ? 96 : 0);
        dma16(vt + off.v0 + rows * npk * T::VES, vst + i * NT * 16 + w * 1024);
    }
}

// Work decomposition shared by the fused kernel and the Q.K^T dump: a
// workgroup of WAVES waves owns (sequence, kv head, head group, query tile);
// wave w takes query head head0 + w % hpw and rows q0 .. q0+31.
struct Work {
    SeqInfo si;
    int s;                    // index of the sequence in the launch's table
    int hkv, head, q0;        // q0 = first query row of this wave
    int head0, hpw;           // first query head of the workgroup, heads per workgroup
    int wg_row0;              // first query row of the workgroup's tile
    int t0;                   // first key tile of the workgroup's split (0 unsplit)
    int nt_wg, nt_w;          // end (exclusive) of the key tiles of the workgroup /
                              // of this wave; tiles t0 .. end-1 are processed
    int split;                // split index of the key range (0 unsplit)
};

template <int WAVES>
__device__ inline int wg_count(const KParams& P, int nq) {
    const int hpw = heads_per_wg(P.group);
    const int rows = 32 * WAVES / hpw;
    return P.hkv * (P.group / hpw) * ((nq + rows - 1) / rows);
}

template <int WAVES>
__device__ inline Work decode_work(const KParams& P) {
    Work w;
    const int hpw = heads_per_wg(P.group);
    const int rows = 32 * WAVES / hpw;
    const int nhg = P.group / hpw;
    int local;
    auto per = [&](int s) {
        return wg_count<WAVES>(P, P.tab.uniform ? P.tab.nq[0] : P.tab.nq[s]) * P.nsplit;
    };
    const int s = find_seq(P, blockIdx.x, per, &local);
    w.s = s;
    w.si = seq_info(P, s);
    const int nq = w.si.nq, nkv = w.si.nkv;
    // a split key range: the split index is the slowest
    const int base = wg_count<WAVES>(P, nq);
    w.split = local / base;
    local %= base;
    // kv head fastest (consecutive workgroups land on different XCDs), then the
    // head group, then query tiles from the heaviest (last) to the lightest
    w.hkv = local % P.hkv;
    const int rest = local / P.hkv;
    const int hg = rest % nhg;
    const int qt_rev = rest / nhg;
    const int nqt = (nq + rows - 1) / rows;
    const int qt = nqt - 1 - qt_rev;
    const int wave = threadIdx.x >> 6;
    const int hw = wave % hpw, rw = wave / hpw;
    w.head0 = w.hkv * P.group + hg * hpw;
    w.hpw = hpw;
    w.head = w.head0 + hw;
    const int wg_row0 = qt * rows;
    w.wg_row0 = wg_row0;
    w.q0 = wg_row0 + rw * 32;
    const int wg_last = min(wg_row0 + rows, nq) - 1;
    const int end_wg = P.causal ? min(nkv, wg_last + nkv - nq + 1) : nkv;
    w.nt_wg = end_wg > 0 ? (end_wg + KVT - 1) / KVT : 0;
    if (w.q0 < nq) {
        const int w_last = min(w.q0 + 31, nq - 1);
        const int end_w = P.causal ? min(nkv, w_last + nkv - nq + 1) : nkv;
        w.nt_w = end_w > 0 ? (end_w + KVT - 1) / KVT : 0;
    } else {
        w.nt_w = 0;
    }
    w.t0 = 0;
    if (P.kv_tiles > 0) {
        w.t0 = w.split * P.kv_tiles;
        const int t1 = w.t0 + P.kv_tiles;
        w.nt_wg = min(w.nt_wg, t1);
        w.nt_w = min(w.nt_w, t1);
    }
    return w;
}

// The wave's Q codes in MFMA B layout: lane (row = lane%32, half = lane/32)
// holds channels [32c + 16*half, +16) for every 32-channel chunk c.
template <int D>
__device__ inline void load_q(const int8_t* qrow, v4i* qf) {
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        qf[c] = *reinterpret_cast<const v4i*>(qrow + 32 * c + 16 * h);
}

// Q quantized in the fused kernel (the pre-pass then skips Q; only where Q
// is not smoothed): q_load reads the lane's values of its row, channels
// [32c + 16*half, +16) for each 32-channel chunk c as load_q reads their
// codes (rows past nq read as 0); q_values converts them and returns the
// lane's absmax.  q_codes then forms the codes with the
// block's absmax a exactly as the pre-pass does: inv = 127/a (both scaled
// by 2^64 first below 2^-100), code = clamp(rne(x*inv), +-127).
template <int DT>
__device__ inline float q_h2f(uint16_t u) {
    if constexpr (DT == 0) return __half2float(__ushort_as_half(u));
    else return __uint_as_float((uint32_t)u << 16);
}

template <int D>
__device__ inline void q_load(const uint16_t* row, bool valid, uint4 (&raw)[D / 32][2]) {
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g)
            raw[c][g] = valid ? *reinterpret_cast<const uint4*>(row + 32 * c + 16 * h + 8 * g)
                              : make_uint4(0u, 0u, 0u, 0u);
}

template <int D, int DT>
__device__ inline float q_values(const uint4 (&raw)[D / 32][2], float (&x)[D / 32][16]) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint32_t wd[4] = {raw[c][g].x, raw[c][g].y, raw[c][g].z, raw[c][g].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float lo = q_h2f<DT>((uint16_t)(wd[k] & 0xffff));
                const float hi = q_h2f<DT>((uint16_t)(wd[k] >> 16));
                x[c][8 * g + 2 * k] = lo;
                x[c][8 * g + 2 * k + 1] = hi;
                m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
            }
        }
    return m;
}

template <int D>
__device__ inline void q_codes(const float (&x)[D / 32][16], float a, v4i* qf) {
    const float rs = a < 0x1p-100f ? 0x1p64f : 1.0f;
    const float inv = a > 0.0f ? 127.0f / (a * rs) : 0.0f;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t wd = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float q = rintf((x[c][4 * j + e] * rs) * inv);
                q = fminf(fmaxf(q, -127.0f), 127.0f);
                wd |= ((uint32_t)(int32_t)q & 0xffu) << (8 * e);
            }
            qf[c][j] = (int)wd;
        }
}

__device__ inline float wave_max64(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// S^T of one 128-key tile: sacc[b] covers keys 32b..32b+31; lane (row,
// half) receives keys 32b + 16*half + r in register r (r = 0..15).  The
// accumulators start at the bits of 1.5*2^23 (sbias_init), so that the int32
// result read as a float is exactly 1.5*2^23 + S.  k_ops reads the A operands
// of one 32-channel chunk (one 16-byte LDS read per 32-key block), qk_chunk
// issues its four MFMAs; chunk-major order keeps consecutive MFMAs
// independent.
__device__ inline void sbias_init(v16i* sacc) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[b][r] = SBIAS_I;
}

template <int D>
__device__ inline void k_ops(const uint8_t* Ks, int c, v4i* a) {
    using T = Tile<D>;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, i = lane & 31;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int row = 32 * b + i;
        a[b] = *reinterpret_cast<const v4i*>(Ks + row * T::KRS +
                                             (((2 * c + h) ^ swz<T::KRS>(row)) << 4));
    }
}

__device__ inline void qk_chunk(const v4i* a, v4i q, v16i* sacc) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
        sacc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[b], q, sacc[b], 0, 0, 0);
}

template <int D>
__device__ inline void qk_tile(const uint8_t* Ks, const v4i* qf, v16i* sacc) {
    sbias_init(sacc);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        v4i a[4];
        k_ops<D>(Ks, c, a);
        qk_chunk(a, qf[c], sacc);
    }
}

// acc[c] += V^T(channels 32c..32c+31) . P^T for one 128-key tile held in a V
// stage (two 64-key halves: P bytes pb[kh]).  v_op reads the A operand of
// half kh, chunk c: two 16-byte granules of the lane's channel row.
template <int D>
__device__ inline v8i v_op(const uint8_t* Vs, int kh, int c) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, qi = lane & 31;
    const int ch = 32 * c + qi;
    const uint8_t* vr = Vs + ch * KVT;
    const int sw = swz<128>(ch);
    const v4i lo = *reinterpret_cast<const v4i*>(vr + (((4 * kh + h) ^ sw) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(vr + (((4 * kh + 2 + h) ^ sw) << 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ inline v16f pv_mfma(v8i a, v8i p, v16f acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, acc, 0, 0, 0, 0, 0, 0);
}

template <int D>
__device__ inline void pv_tile(const uint8_t* Vs, const v8i* pb, v16f* acc) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) acc[c] = pv_mfma(v_op<D>(Vs, kh, c), pb[kh], acc[c]);
}

// The 16-bit variant: acc[c] += V^T(channels 32c..32c+31) . P^T with the
// 32x32x16 f16 / bf16 MFMA.  Step (b, j) sums 16 keys: lane half h supplies
// keys 32b + 16h + 8j .. +7 of both operands (the summation index only has
// to agree between them), V^T as one 16-byte granule of its 256-byte row and
// P as ph[2b + j].
template <int D, int DT>
__device__ inline void pv_tile_h(const uint8_t* Vs, const v4i* ph, v16f* acc) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, qi = lane & 31;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // one 32-key block at a time keeps the operand reads in flight (and
        // their registers) to one block's worth
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const int ch = 32 * c + qi;
                const int g = 4 * b + 2 * h + j;
                const v4i a = *reinterpret_cast<const v4i*>(Vs + ch * (2 * KVT) +
                                                            ((g ^ swz<256>(ch)) << 4));
                if constexpr (DT == 0)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, ph[2 * b + j]), acc[c],
                        0, 0, 0);
                else
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, ph[2 * b + j]),
                        acc[c], 0, 0, 0);
            }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Two FP32 values rounded to nearest even into the 16-bit type DT (0 fp16,
// 1 bf16), packed low | high << 16.
// (one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 per pair)
template <int DT>
__device__ inline uint32_t pack16(float lo, float hi) {
    const v2f x = {lo, hi};
    if constexpr (DT == 0) return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2h));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
}

__device__ inline float swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The tile's row maximum m (log2 units), raised where its magnitude is large.
// The largest exponent of a row, x = S*c - (m - log2 448), can exceed log2 448
// by the FP32 roundings of m (a product), of m - log2 448 and of the
// exponent's FMA: up to three units in the last place of m.  Below |m| = 2^16
// that is under 0.024, and 2^x stays below 464, where v_cvt_pk_fp8_f32 turns
// from the top code 448 to the NaN code; above, it could reach the NaN code
// (and, with a 16-bit P, whose exponent has no 448 in it, p could overflow
// once the unit in the last place of m is large).
// There m is raised by 6 * 2^-23 * (|m| - 2^16), at least three units in its
// last place from 2^17 on, which keeps every exponent at or below log2 448:
// the softmax is the same for any m at or above the row's largest score, and
// the rescale factors, l and the LSE follow the raised m.  Below 2^16 the
// raise is exactly 0 (m unchanged); a row with no visible key yet (m = -inf)
// keeps -inf (the clamp of d to 2^100).  Three VALU instructions per tile.
__device__ inline float raise_max(float m) {
    const float d = __builtin_amdgcn_fmed3f(fabsf(m) - 65536.0f, 0.0f, 0x1p100f);
    return fmaf(d, 6.0f * 0x1p-23f, m);
}

// Online softmax of one tile, in two halves so that the fused kernel can run
// them in different phases.
//
// The score half (score_exp) turns the tile's biased int32 scores into
// p = 2^(s*log2 e - m) in FP32 (the FP8 operand's static scale 448 is folded
// into the exponent; the 16-bit operand has none), updates the running max m
// and returns alpha, the factor that moves earlier contributions to the new
// max.  Keys past `lim` are masked when MASK.  Score scales: with 64-token K
// blocks c0 serves the tile's first 64 keys and c1 the rest; with 32-token
// blocks (QB = 32) c0..c3 serve the four 32-key blocks.
//
// The operand half adds the tile's FP32 p to the running sum,
// l = alpha*l + sum p (row_sum), and writes P^ in the B layout of the
// 32x32x64 FP8 MFMA (half kh covers the lane's keys of blocks 2kh and 2kh+1,
// bytes 0..15 and 16..31) -- or, with 16-bit operands (PVH), p itself
// rounded into the type DT, eight keys per ph entry as pv_tile_h reads them
// (pack_p).
// PRESUB: the scores in sacc are already exact (the bias subtracted in the
// MFMA phase, as float bits).
template <bool MASK, bool HAS_DS, bool PVH = false, int QB = QBLK, bool PRESUB = false>
__device__ inline float score_exp(v16i* sacc, float (&p)[4][16], float c0, float c1, float c2,
                                  float c3, const float* dsl, float sml2, int kt0, int lim,
                                  float& m_run) {
    constexpr float SB = PRESUB ? 0.0f : SBIAS_F;
    constexpr float POFF = PVH ? 0.0f : LOG2_448;
    auto cof = [&](int b) {
        if constexpr (QB == 32) return b == 0 ? c0 : (b == 1 ? c1 : (b == 2 ? c2 : c3));
        else return b < 2 ? c0 : c1;
    };
    const int h = (threadIdx.x & 63) >> 5;
    // key kt0 + 32b + r is masked when 32b + r > lim - kt0: one compare with
    // a constant per key
    const int th = lim - kt0;
    float m_new;
    if constexpr (!HAS_DS) {
        if constexpr (MASK) {
            // masked keys get the bits of -inf: as integers below every
            // biased score, as floats they give 2^-inf = 0 below (c > 0)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sacc[b][r] = 32 * b + r > th ? NEG_INF_BITS : sacc[b][r];
        }
        // the exact scores first (one subtraction each, independent of the
        // row maximum), then three-input float max trees, one per block of
        // keys that shares a scale, then the exponent's FMA
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                p[b][r] = PRESUB ? __int_as_float(sacc[b][r]) : __int_as_float(sacc[b][r]) - SB;
        auto fmax16 = [&](int b) {
            float l1[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) l1[i] = fmaxf(fmaxf(p[b][3 * i], p[b][3 * i + 1]), p[b][3 * i + 2]);
            return fmaxf(fmaxf(fmaxf(l1[0], l1[1]), l1[2]), fmaxf(fmaxf(l1[3], l1[4]), p[b][15]));
        };
        float fm;
        if constexpr (QB == 32) {
            fm = -INFINITY;
#pragma unroll
            for (int b = 0; b < 4; ++b) fm = fmaxf(fm, fmax16(b) * cof(b));
        } else {
            fm = fmaxf(fmaxf(fmax16(0), fmax16(1)) * c0, fmaxf(fmax16(2), fmax16(3)) * c1);
        }
        // (raised per lane before the two halves of the row meet: the raise
        // grows with m, so the row's maximum is raised as a whole)
        m_new = fmaxf(m_run, swap_max(raise_max(fm)));
        const float nm = POFF - (m_new == -INFINITY ? 0.0f : m_new);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) p[b][r] = __builtin_amdgcn_exp2f(fmaf(p[b][r], cof(b), nm));
    } else {
        // here c0, c1 leave out sm_scale*log2(e): y = S*sq*sk + dS is formed
        // first (its maximum taken), and the base-2 factor is applied inside
        // the exponent's FMA
        float mt = -INFINITY;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float c = cof(b);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float sv = PRESUB ? __int_as_float(sacc[b][r]) : __int_as_float(sacc[b][r]) - SB;
                float y = fmaf(sv, c, dsl[32 * b + 16 * h + r]);
                if (MASK) y = 32 * b + r > th ? -INFINITY : y;
                p[b][r] = y;
                mt = fmaxf(mt, y);
            }
        }
        m_new = fmaxf(m_run, swap_max(raise_max(mt * sml2)));
        const float nm = POFF - (m_new == -INFINITY ? 0.0f : m_new);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) p[b][r] = __builtin_amdgcn_exp2f(fmaf(p[b][r], sml2, nm));
    }
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    return alpha;
}

// l = alpha*l + (sum of the tile's FP32 p), in NPS interleaved partial sums
// (16 shortens the dependency chains; measured faster at d = 64, where the
// softmax is the whole bound, and not at d = 128).
template <int NPS = 8>
__device__ inline void row_sum(const float (&p)[4][16], float alpha, float& l_run) {
    float ps[NPS];
#pragma unroll
    for (int k = 0; k < NPS; ++k) ps[k] = p[0][k];
    if constexpr (NPS == 16) {
#pragma unroll
        for (int b = 1; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) ps[r] += p[b][r];
#pragma unroll
        for (int k = 0; k < 8; ++k) ps[k] += ps[k + 8];
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (b > 0 || r >= 8) ps[r % 8] += p[b][r];
    }
    const float psum = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    l_run = fmaf(alpha, l_run, psum);
}

// The P operand of one tile from its FP32 p.
template <bool PVH = false, int DT = 0>
__device__ inline void pack_p(const float (&p)[4][16], v8i* pb, v4i* ph) {
    if constexpr (PVH) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int wd = 0; wd < 4; ++wd)
                    ph[2 * b + j][wd] =
                        (int)pack16<DT>(p[b][8 * j + 2 * wd], p[b][8 * j + 2 * wd + 1]);
    } else {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int wd = 0; wd < 8; ++wd) {
                const int b = 2 * kh + wd / 4, r0 = 4 * (wd % 4);
                // the first convert fills the low half of the word and the
                // second the high half, so the word's prior contents do not
                // matter: it is seeded with a value that dies here (no zeroing
                // move)
                uint32_t u = e4m3_pk<false>(p[b][r0], p[b][r0 + 1], __float_as_uint(p[b][r0]));
                u = e4m3_pk<true>(p[b][r0 + 2], p[b][r0 + 3], u);
                pb[kh][wd] = (int)u;
            }
    }
}

// The whole online softmax of one tile (both halves in one place).
template <bool MASK, bool HAS_DS, bool PVH = false, int DT = 0, int QB = QBLK, int NPS = 8,
          bool PRESUB = false>
__device__ inline float softmax_tile(v16i* sacc, v8i* pb, v4i* ph, float c0, float c1, float c2,
                                     float c3, const float* dsl, float sml2, int kt0, int lim,
                                     float& m_run, float& l_run) {
    float p[4][16];
    const float alpha = score_exp<MASK, HAS_DS, PVH, QB, PRESUB>(sacc, p, c0, c1, c2, c3, dsl,
                                                                 sml2, kt0, lim, m_run);
    row_sum<NPS>(p, alpha, l_run);
    pack_p<PVH, DT>(p, pb, ph);
    return alpha;
}

template <int D>
__device__ inline void rescale(v16f* acc, float alpha) {
    if (!__all(alpha == 1.0f)) {
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[c][r] *= alpha;
    }
}

// One MFMA phase of the FP8 path: acc = alpha*acc + V^T.P^T of the previous
// tile (when pv), then S = Q.K^T of this tile into sacc.  The LDS operand reads
// run ahead of the matrix instructions that consume them (two P.V
// instructions, two Q.K chunks), so that their latency passes under earlier
// matrix work instead of being waited for at every pair of reads; K chunk 0
// is read first and arrives under the P.V.  With DEFER the previous tile's
// P operand and row sum are formed here too, from its FP32 p in pd.  `mid`
// runs between the P.V and the Q.K^T instructions (before the score
// accumulators are live).
template <int D, bool DEFER, int NPS, typename Mid>
__device__ inline void mfma_phase(const uint8_t* Vs, const uint8_t* Ks, bool pv, v8i* pb,
                                  const float (&pd)[4][16], v16i* sacc, v16f* acc, const v4i* qf,
                                  float alpha, float& l_run, Mid mid) {
    constexpr int NC = D / 32;
    constexpr int NPV = 2 * NC;                // P.V instructions, kh-major
    v4i ka[NC][4];
    k_ops<D>(Ks, 0, ka[0]);
    if (pv) {
        v8i va[NPV];
        va[0] = v_op<D>(Vs, 0, 0);
        va[1] = v_op<D>(Vs, 1 / NC, 1 % NC);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DEFER) pack_p<false, 0>(pd, pb, nullptr);
        rescale<D>(acc, alpha);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + 2 < NPV) va[i + 2] = v_op<D>(Vs, (i + 2) / NC, (i + 2) % NC);
            __builtin_amdgcn_sched_barrier(0);
            acc[i % NC] = pv_mfma(va[i], pb[i / NC], acc[i % NC]);
        }
        if constexpr (DEFER) row_sum<NPS>(pd, alpha, l_run);
    }
    mid();
    if constexpr (NC > 1) k_ops<D>(Ks, 1, ka[1]);
    __builtin_amdgcn_sched_barrier(0);
    sbias_init(sacc);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) k_ops<D>(Ks, c + 2, ka[c + 2]);
        __builtin_amdgcn_sched_barrier(0);
        qk_chunk(ka[c], qf[c], sacc);
    }
}

// ---------------------------------------------------------------------------
// Per-block Q smoothing (SageAttention2 summary, "Main concepts" item 2: Q is
// smoothed by its channel mean; here one mean per Q quantization block).  A
// workgroup's rows form NPAIR (query head, Q block) pairs: pair p is head
// slot p % hpw and block p / hpw of the workgroup's row tile.  The scores of
// pair p owe ds_seq_j + (mu_b - mu_q).k_j: the sequence's compensation
// ds_seq (the per-head bias stage, copied from the pre-pass) plus the block's
// deviation, formed here from its 15-bit code (128*hi + lo, one FP32 scale)
// and the INT8 key codes of the tile with v_mfma_i32_16x16x64_i8.  The
// codes sit in a 16-row LDS table (row p: hi of pair p, row 8 + p: lo), and
// each tile's compensations in a per-pair bias stage (two, alternating).
// ---------------------------------------------------------------------------
template <int QB>
struct Bqs {
    static constexpr int NPAIR = 256 / QB;          // pairs of a workgroup (4 or 8)
    static constexpr int STAGE = NPAIR * KVT * 4;   // bytes of one per-pair bias stage
    static constexpr int TROW = 128;                // table bytes per code row
    static constexpr int TABLE = 16 * TROW;
    static constexpr int BYTES = 2 * STAGE + TABLE + 64;   // + 8 scales (padded)
};

// Index of (sequence, head, Q block) in the per-block pre-pass arrays.
__device__ inline int64_t qblock_index(const KParams& P, const SeqInfo& si, int head, int qb_len,
                                       int gblk) {
    return (si.rq * P.hq + (int64_t)head * si.npq) / qb_len + gblk;
}

// Load the workgroup's code table and scales into LDS (threads 0..135).
// Pairs past NPAIR, blocks past the padded sequence and channels past D are
// zero (their products vanish).
template <int D, int QB>
__device__ inline void bqs_load(const KParams& P, const Work& w, const int8_t* mcode,
                                const float* mcs, uint8_t* tab, float* tsc) {
    using B = Bqs<QB>;
    const int tid = threadIdx.x;
    const SeqInfo& si = w.si;
    auto pair_index = [&](int p, int64_t* ib) {
        if (p >= B::NPAIR) return false;
        const int gblk = w.wg_row0 / QB + p / w.hpw;
        if (gblk * QB >= si.npq) return false;
        *ib = qblock_index(P, si, w.head0 + p % w.hpw, QB, gblk);
        return true;
    };
    if (tid < 128) {
        const int row = tid >> 3, g = tid & 7;
        v4i val = {0, 0, 0, 0};
        int64_t ib;
        if (16 * g < D && pair_index(row & 7, &ib))
            val = *reinterpret_cast<const v4i*>(mcode + ib * 2 * D + (row >> 3) * D + 16 * g);
        *reinterpret_cast<v4i*>(tab + row * B::TROW + 16 * g) = val;
    } else if (tid < 136) {
        int64_t ib;
        tsc[tid - 128] = pair_index(tid - 128, &ib) ? mcs[ib] : 0.0f;
    }
}

// The per-pair compensations of one key tile, by the four waves of group 0:
// wave wi covers the tile's LDS rows 32wi .. 32wi+31 in two 16-row MFMA
// tiles, for every pair at once (B columns 0..7: hi codes, 8..15: lo codes).
// bqs_mfma issues the matrix instructions and bqs_store combines and writes
// the results (where in the MFMA phase: see the fused kernel).  The 16x16
// result gives lane (column c, k-group g) the rows 4g .. 4g+3 of its tile
// for column c; the lo sum of pair c comes from the lane 8 columns over (a
// DPP rotation by 8 within the 16-lane row).
// Rows 4g .. 4g+3 hold four consecutive keys (key_of_row), written as one
// float4.  The deviation term is fl32(fl32(T) * fl32(s_mu * s_k)), added to
// ds_seq without contraction.
template <int D, int QB>
__device__ inline void bqs_mfma(const uint8_t* Ks, const uint8_t* tab, v4i* acc) {
    using T = Tile<D>;
    using B = Bqs<QB>;
    constexpr int NS = (D + 63) / 64;               // 64-channel steps
    // (at d = 128 the thread index passes through an empty asm so that the
    // addresses below are formed here on every tile rather than hoisted out
    // of the loop, where they would hold registers through the whole kernel)
    int tid = threadIdx.x;
    if constexpr (D == 128) asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wi = (tid >> 6) & 3;
    const int col = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[m] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int g = 4 * s + kg;                   // 16-channel granule
        const v4i b = *reinterpret_cast<const v4i*>(tab + col * B::TROW + 16 * g);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int row = 32 * wi + 16 * m + col; // A row of this lane
            const v4i a = *reinterpret_cast<const v4i*>(Ks + row * T::KRS +
                                                        ((g ^ swz<T::KRS>(row)) << 4));
            acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[m], 0, 0, 0);
        }
    }
}

// kst: the tile's key-block scales in global memory.
template <int D, int QB>
__device__ inline void bqs_store(const v4i* acc, const float* hds, float* pst, const float* tsc,
                                 const float* kst, int hpw) {
#pragma clang fp contract(off)
    using B = Bqs<QB>;
    int tid = threadIdx.x;                          // (d = 128: not hoisted, as in bqs_mfma)
    if constexpr (D == 128) asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wi = (tid >> 6) & 3;
    const int col = lane & 15, kg = lane >> 4;
    int lo[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo[m][i] = __builtin_amdgcn_mov_dpp(acc[m][i], 0x128, 0xf, 0xf, false);   // row_ror:8
    if (col < B::NPAIR) {
        const float smu = tsc[col];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int kk = key_of_row(32 * wi + 16 * m + 4 * kg);
            const float ks = kst[kk / QB];
            const float f = smu * ks;
            // (16-byte integer accesses, as the operand reads: typed float
            // accesses make the compiler wait here for the phase's copies)
            const v4i base = *reinterpret_cast<const v4i*>(hds + (col % hpw) * KVT + kk);
            v4i out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float corr = (float)(acc[m][i] * 128 + lo[m][i]) * f;
                out[i] = __float_as_int(__int_as_float(base[i]) + corr);
            }
            *reinterpret_cast<v4i*>(pst + col * KVT + kk) = out;
        }
    }
}

template <int DT>
__device__ inline uint32_t f2h_bits(float f) {
    if constexpr (DT == 0) {
        return (uint32_t)__half_as_ushort(__float2half_rn(f));
    } else {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
        u += 0x7fffu + ((u >> 16) & 1u);
        return u >> 16;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// The fused forward kernel (8 waves, ping-pong between two groups of 4).
//
// Barrier epochs: group 0 runs [MFMA(t)] bar [softmax(t)] bar for t = 0, 1, ...;
// group 1 runs the same after one extra leading barrier, so in every epoch one
// group is in its MFMA phase and the other in its softmax phase.
// MFMA(t) = acc = alpha(t-1) * acc + V(t-1)^T . P^(t-1)^T, then S(t) = Q.K(t)^T;
// softmax(t) produces P^(t) and the alpha(t) that acc owes before the next P.V.
// LDS lifetimes (epochs 2t, 2t+1 read K(t) and V(t-1); softmax(t) of group 1
// runs in epoch 2t+2 and reads the score bias of tile t):
//   K(t+1), V(t): copied at the start of MFMA(t) by each group (epochs 2t,
//   2t+1) into the buffers freed by K(t-1), V(t-2) (last read in 2t-2, 2t-1);
//   every wave waits for its copies before each barrier.
//   bias(t): three buffers, as it is read up to epoch 2t+2.
// ---------------------------------------------------------------------------
// With BQS (per-block Q smoothing; implies HAS_DS and the FP8 P.V), group 0
// also forms each tile's per-pair compensations at the start of its MFMA
// phase, from the tile's K codes and per-head bias stage (both complete at
// that point); the softmax phases of both groups read them from the per-pair
// stage of the tile (two stages: tile t is written in epoch 2t and read in
// epochs 2t+1 and 2t+2).
// Dynamic LDS of the fused kernel: K and V^T double buffers, the score-bias
// stages and the per-block Q smoothing area (the kernel's own Q quantization
// adds 64 bytes of slots after it).
template <int D, bool HAS_DS, bool PVH, bool BQS = false, int QB = QBLK>
constexpr int lds_bytes() {
    return 2 * Tile<D, PVH>::KBYTES + 2 * Tile<D, PVH>::VBYTES +
           (HAS_DS ? 3 * Tile<D, PVH>::DSBYTES : 0) + (BQS ? Bqs<QB>::BYTES : 0);
}

template <int D, int DT, bool HAS_DS, bool PVH, int QB, bool DUMP = false, bool BQS = false>
__global__ __launch_bounds__(FWD_NT) void k_attn(KParams P, const int8_t* __restrict__ qc,
                                                 const float* __restrict__ qsc,
                                                 const int8_t* __restrict__ kc,
                                                 const float* __restrict__ ksc,
                                                 const uint8_t* __restrict__ vc,
                                                 const float* __restrict__ vsc,
                                                 const float* __restrict__ ds,
                                                 const float* __restrict__ mu_v,
                                                 uint16_t* __restrict__ o,
                                                 float* __restrict__ lse,
                                                 const int8_t* __restrict__ mcode,
                                                 const float* __restrict__ mcs) {
    static_assert(!BQS || (HAS_DS && !PVH && !DUMP), "per-block Q smoothing: FP8 P.V with bias");
    extern __shared__ __align__(16) uint8_t smem[];
    using T = Tile<D, PVH>;
    const Work w = decode_work<FWD_WAVES>(P);
    const SeqInfo& si = w.si;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, qi = lane & 31;
    const int grp = (threadIdx.x >> 6) >> 2;
    const int my_q = w.q0 + qi;
    const int nq = si.nq, nkv = si.nkv;

    const int64_t krow0 = (si.rk * P.hkv + (int64_t)w.hkv * si.npk);
    const int8_t* kbase = kc + krow0 * D;
    const uint8_t* vbase = vc + krow0 * D * T::VES;
    const float* kscb = ksc + krow0 / QB;
    const float* dsb = HAS_DS ? ds + si.rk * P.hq + (int64_t)w.head0 * si.npk : nullptr;

    v4i qf[D / 32];
    float sq = 0.0f;
    // With raw Q the kernel quantizes it here (q_values, q_codes): every wave
    // posts the absmax of its 32 rows to an LDS slot, and a 64-token block
    // takes the larger of its two waves' after the first barrier below (so
    // every wave posts, whether or not it has key tiles).
    // (compiled only where Q is not smoothed: with the score bias the
    // prologue measured slower than the pre-pass work it saves)
    const bool qraw = !DUMP && !BQS && !HAS_DS && P.q_raw != nullptr;
    float qx[D / 32][16];
    uint4 qraw_v[D / 32][2];
    float* qslot = reinterpret_cast<float*>(smem + lds_bytes<D, HAS_DS, PVH, BQS, QB>());
    if (qraw) {
        // (the loads go out here; their values are first used after the
        // first K tile's copies are issued, so the two latencies overlap)
        const uint16_t* row = P.q_raw + si.q_el + (int64_t)w.head * P.qs.h +
                              (int64_t)min(my_q, nq - 1) * P.qs.n;
        q_load<D>(row, my_q < nq, qraw_v);
    } else if (w.nt_w > w.t0) {
        const int64_t qrow0 = si.rq * P.hq + (int64_t)w.head * si.npq;
        load_q<D>(qc + (qrow0 + my_q) * D, qf);
        if constexpr (!DUMP) sq = qsc[(qrow0 + w.q0) / QB];
    } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c] = v4i{0, 0, 0, 0};
    }

    v16f acc[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const int diag = my_q + nkv - nq;          // last visible key of this row (causal)
    const int wave_diag = w.q0 + nkv - nq;     // ... of the wave's first row
    const int lim = P.causal ? min(diag, nkv - 1) : nkv - 1;

    uint8_t* kst0 = smem;
    uint8_t* vst0 = smem + 2 * T::KBYTES;
    uint8_t* dst0 = vst0 + 2 * T::VBYTES;      // score-bias stages (HAS_DS)
    uint8_t* bq0 = dst0 + 3 * T::DSBYTES;      // per-pair stages, code table, scales (BQS)
    uint8_t* btab = bq0 + 2 * Bqs<QB>::STAGE;
    float* btsc = reinterpret_cast<float*>(btab + Bqs<QB>::TABLE);
    const int my_pair = (32 * ((threadIdx.x >> 6) / w.hpw)) / QB * w.hpw + (threadIdx.x >> 6) % w.hpw;
    DmaOffsets<D, FWD_NT, PVH> off;
    off.init(si.npk);

    // The epilogue's V scales (and V means) of the kv head: copied into LDS
    // here, behind the 64 bytes of Q absmax slots, so that the epilogue reads
    // them there instead of waiting on memory after the last tile (the
    // 16-bit P.V has no V scale).
    float* vslds = reinterpret_cast<float*>(smem + lds_bytes<D, HAS_DS, PVH, BQS, QB>() + 64);
    const int64_t vsb = ((int64_t)si.sid * P.hkv + w.hkv) * D;
    if constexpr (!DUMP) {
        const int wave = threadIdx.x >> 6;
        if (!PVH && wave == 0 && lane < D / 4)
            dma16(vsc + vsb + 4 * lane, reinterpret_cast<uint8_t*>(vslds));
        if (mu_v && wave == 1 && lane < D / 4)
            dma16(mu_v + vsb + 4 * lane, reinterpret_cast<uint8_t*>(vslds + D));
    }

    // stage the first tile (K and bias) with every wave, then offset group 1.
    // Stage buffers are chosen by the tile's place r = t - t0 in the split.
    if (w.nt_wg > w.t0)
        stage_k<D, FWD_NT, HAS_DS, PVH>(kst0, dst0, off, kbase, dsb, si.npk, w.t0, w.hpw);
    if constexpr (BQS) bqs_load<D, QB>(P, w, mcode, mcs, btab, btsc);
    if (qraw) {
        const float m = wave_max64(q_values<D, DT>(qraw_v, qx));
        if (lane == 0) qslot[threadIdx.x >> 6] = m;
    }
    bar();
    if (qraw) {
        const int wave = threadIdx.x >> 6;
        float a = qslot[wave];
        if constexpr (QB == 64) a = fmaxf(a, qslot[((wave / w.hpw) ^ 1) * w.hpw + wave % w.hpw]);
        q_codes<D>(qx, a, qf);
        sq = a > 0.0f ? a / 127.0f : 0.0f;
    }
    if (grp == 1) bar();

    v8i pb[2];                  // P^ of the previous tile (E4M3)
    v4i ph[PVH ? 8 : 1];        // ... or its 16-bit p (PVH)
    constexpr int NPS = D == 64 ? 16 : 8;
    // Where a tile's row sum and P operand are formed.  At d = 64 the matrix
    // phase is short and the softmax phase is the whole bound: they move to
    // the next MFMA phase, under the P.V and Q.K matrix instructions.  At
    // d = 96 and 128 the MFMA phase is as long as the softmax phase already,
    // and they stay in the softmax phase.
    constexpr bool DEFER = D == 64 && !PVH;
    // software-pipelined LDS operand reads in the MFMA phase (FP8 path)
    constexpr bool PIPE = true;
    // With the score bias at d = 128, the exact scores (the accumulator bias
    // subtracted) are formed at the end of the MFMA phase, in place, where
    // the waves wait at the barrier, instead of in the softmax phase (3%
    // faster there; without the bias it measured 3% slower on causal_gqa and
    // neutral on llm_prefill and at d = 96).
    constexpr bool PRESUB = !PVH && !DUMP && HAS_DS && D == 128;
    v16i sacc[4];               // a tile's biased int32 scores (Q.K^T)
    float pd[4][16];            // with DEFER: the previous tile's FP32 p (else unused)
    float alpha_prev = 1.0f;   // rescale owed to acc before its next P.V
    // the P.V of the previous tile (its place rr in the split)
    auto pv_prev = [&](int rr) {
        if constexpr (DEFER) pack_p<PVH, DT>(pd, pb, ph);
        rescale<D>(acc, alpha_prev);
        const uint8_t* vs_ = vst0 + (rr & 1) * T::VBYTES;
        if constexpr (PVH) pv_tile_h<D, DT>(vs_, ph, acc);
        else pv_tile<D>(vs_, pb, acc);
        if constexpr (DEFER) row_sum<NPS>(pd, alpha_prev, l_run);
    };

    constexpr int NB = KVT / QB;             // key blocks of a tile (2 or 4)
    for (int t = w.t0; t < w.nt_wg; ++t) {
        const int r = t - w.t0;
        // ---- MFMA phase ----
        __builtin_amdgcn_s_setprio(2);
        // BQS: group 0 forms the tile's per-pair compensations.  d = 128 has
        // no registers to hold the sums through the P.V, and does all of it
        // before the phase's copies are issued (so that its reads do not wait
        // for them); d = 64 and 96 issue the matrix instructions here and
        // store the results between the P.V and the Q.K^T.
        constexpr bool BQS_EARLY = D == 128;
        v4i bacc[2];
        auto bqs_fin = [&]() {
            if constexpr (BQS) {
                if (grp == 0)
                    bqs_store<D, QB>(bacc,
                                  reinterpret_cast<const float*>(dst0 + (r % 3) * T::DSBYTES),
                                  reinterpret_cast<float*>(bq0 + (r & 1) * Bqs<QB>::STAGE), btsc,
                                  kscb + NB * t, w.hpw);
            }
        };
        DmaOffsets<D, FWD_NT, PVH> offt = off;
        if constexpr (BQS && BQS_EARLY) {
            if (grp == 0) bqs_mfma<D, QB>(kst0 + (r & 1) * T::KBYTES, btab, bacc);
            bqs_fin();
        }
        // at d = 128 with the block bias or with 16-bit P and the score bias,
        // the copies' per-lane addresses are formed on every tile: held
        // through the loop they are what the registers cannot afford, and a
        // reload between the copies waits for them
        if constexpr (D == 128 && (BQS || (PVH && HAS_DS)))
            asm volatile("" : "+v"(offt.k0), "+v"(offt.v0));
        if (t + 1 < w.nt_wg)
            stage_k<D, FWD_NT, HAS_DS, PVH>(kst0 + ((r + 1) & 1) * T::KBYTES,
                                            dst0 + ((r + 1) % 3) * T::DSBYTES, offt, kbase, dsb,
                                            si.npk, t + 1, w.hpw);
        if constexpr (!DUMP)   // (the Q.K^T export reads no V)
            stage_v<D, FWD_NT, PVH>(vst0 + (r & 1) * T::VBYTES, offt, vbase, si.npk, t);
        if constexpr (BQS && !BQS_EARLY) {
            if (grp == 0) bqs_mfma<D, QB>(kst0 + (r & 1) * T::KBYTES, btab, bacc);
        }
        auto bqs_mid = [&]() {
            if constexpr (!BQS_EARLY) bqs_fin();
        };
        if (t < w.nt_w) {
            const uint8_t* ks_ = kst0 + (r & 1) * T::KBYTES;
            if constexpr (PVH || !PIPE) {
                // P.V of the previous tile first: its p then dies before S(t)
                // is formed (needed to fit the registers with 16-bit P)
                if (r > 0) pv_prev(r - 1);
                qk_tile<D>(ks_, qf, sacc);
            } else {
                mfma_phase<D, DEFER, NPS>(vst0 + ((r - 1) & 1) * T::VBYTES, ks_, !DUMP && r > 0,
                                          pb, pd, sacc, acc, qf, alpha_prev, l_run, bqs_mid);
                if constexpr (PRESUB) {
                    // (the empty asm keeps each subtraction here)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            sacc[b][rr] = __float_as_int(__int_as_float(sacc[b][rr]) - SBIAS_F);
                            asm volatile("" : "+v"(sacc[b][rr]));
                        }
                }
            }
        } else {
            if (!DUMP && t == w.nt_w && r > 0) {
                // this wave's rows are done: flush its last tile
                pv_prev(r - 1);
            }
            bqs_mid();
        }
        // the tile's score scales, loaded ahead of the softmax phase (the
        // empty asm keeps the compiler from sinking the loads past the barrier)
        // (a zero scale -- an all-zero block -- is raised to the smallest
        // normal float, which leaves every score unchanged after rounding and
        // keeps a masked key's -inf * c at -inf)
        auto cs = [&](int b) {
            if constexpr (DUMP) return 0.0f;
            const float ks = kscb[NB * t + b];
            return fmaxf(HAS_DS ? sq * ks : sq * ks * P.sml2, FLT_MIN);
        };
        float c0 = cs(0), c1 = cs(1);
        float c2 = NB == 4 ? cs(NB == 4 ? 2 : 0) : 0.0f, c3 = NB == 4 ? cs(NB == 4 ? 3 : 0) : 0.0f;
        asm volatile("" : "+v"(c0), "+v"(c1));
        if constexpr (NB == 4) asm volatile("" : "+v"(c2), "+v"(c3));
        __builtin_amdgcn_s_setprio(0);
        bar();
        // ---- softmax phase ----
        if (DUMP && t < w.nt_w && my_q < nq) {
            // the test export: the exact int32 scores of the tile's keys
            int32_t* out = reinterpret_cast<int32_t*>(o) +
                           (P.tab.uniform ? (int64_t)w.s * P.hq * nq * nkv : P.tab.dump0[w.s]) +
                           ((int64_t)w.head * nq + my_q) * nkv;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = t * KVT + 32 * b + 16 * h + rr;
                    if (j < nkv) out[j] = sacc[b][rr] - SBIAS_I;
                }
        } else if (!DUMP && t < w.nt_w) {
            const int kt0 = t * KVT + 16 * h;     // key of sacc[b][r] = kt0 + 32b + r
            const float* dsl =
                BQS ? reinterpret_cast<const float*>(bq0 + (r & 1) * Bqs<QB>::STAGE) + my_pair * KVT
                : HAS_DS ? reinterpret_cast<const float*>(dst0 + (r % 3) * T::DSBYTES) +
                               (w.head - w.head0) * KVT
                         : nullptr;
            const bool need_mask =
                (t + 1) * KVT > nkv || (P.causal && (t + 1) * KVT - 1 > wave_diag);
            // acc (the tiles before t, at the previous max) is rescaled by
            // alpha in the next MFMA phase, before the P.V of tile t
            if constexpr (DEFER) {
                if (need_mask)
                    alpha_prev = score_exp<true, HAS_DS, PVH, QB, PRESUB>(sacc, pd, c0, c1, c2, c3, dsl,
                                                                  P.sml2, kt0, lim, m_run);
                else
                    alpha_prev = score_exp<false, HAS_DS, PVH, QB, PRESUB>(sacc, pd, c0, c1, c2, c3, dsl,
                                                                   P.sml2, kt0, lim, m_run);
            } else {
                if (need_mask)
                    alpha_prev = softmax_tile<true, HAS_DS, PVH, DT, QB, NPS, PRESUB>(
                        sacc, pb, ph, c0, c1, c2, c3, dsl, P.sml2, kt0, lim, m_run, l_run);
                else
                    alpha_prev = softmax_tile<false, HAS_DS, PVH, DT, QB, NPS, PRESUB>(
                        sacc, pb, ph, c0, c1, c2, c3, dsl, P.sml2, kt0, lim, m_run, l_run);
            }
        }
        bar();
    }
    if (!DUMP && w.nt_w > w.t0 && w.nt_w == w.nt_wg) pv_prev(w.nt_wg - 1 - w.t0);
    if (grp == 0) bar();   // balance group 1's leading barrier
    if constexpr (DUMP) return;

    // epilogue: lanes l and l+32 hold the same row's partial sums.  The
    // wave's 32 output rows are assembled in LDS (rows of RS bytes, 16-byte
    // granules XOR-swizzled by row) and then written as whole rows, 16 bytes
    // per lane.
    const float l_tot = swap_sum(l_run);
    if (P.kv_tiles > 0) {
        // split key range: this split's partial of each row, unnormalised:
        // acc*v_scale + mu_v*l (the mean then comes out of the merge's
        // division by the total l), with m (log2 units) and l
        if (my_q < nq) {
            const int64_t row = si.lse0 + (int64_t)w.head * P.lse_hstride + my_q;
            const int64_t pr = (int64_t)w.split * P.rows_total + row;
            const bool add_mu = mu_v && l_tot > 0.0f;
            float* po = P.part_o + pr * D;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ch0 = 32 * c + 8 * r4 + 4 * h;
                    const float4 s4 = PVH ? make_float4(1.f, 1.f, 1.f, 1.f)
                                          : *reinterpret_cast<const float4*>(vslds + ch0);
                    const float4 m4 = add_mu ? *reinterpret_cast<const float4*>(vslds + D + ch0)
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
                    *reinterpret_cast<float4*>(po + ch0) =
                        make_float4(fmaf(acc[c][4 * r4], s4.x, m4.x * l_tot),
                                    fmaf(acc[c][4 * r4 + 1], s4.y, m4.y * l_tot),
                                    fmaf(acc[c][4 * r4 + 2], s4.z, m4.z * l_tot),
                                    fmaf(acc[c][4 * r4 + 3], s4.w, m4.w * l_tot));
                }
            if (h == 0) *reinterpret_cast<float2*>(P.part_ml + 2 * pr) = make_float2(m_run, l_tot);
        }
        return;
    }
    constexpr int RS = D == 64 ? 128 : 256;    // LDS bytes per staged row
    constexpr int NGR = RS / 16;               // granules per staged row
    static_assert(FWD_WAVES * 32 * RS <= 2 * T::KBYTES + 2 * T::VBYTES, "staging fits the stages");
    __syncthreads();                           // every wave is done with the tile stages
    uint8_t* stg = smem + (threadIdx.x >> 6) * 32 * RS;
    if (w.q0 < nq) {
        const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        // the scales (and means) from their LDS copy; the 16-bit operands
        // carry no scale
        float4 sv[D / 32][4], mv[D / 32][4];
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                sv[c][r4] = PVH ? make_float4(1.f, 1.f, 1.f, 1.f)
                                : *reinterpret_cast<const float4*>(vslds + 32 * c + 8 * r4 + 4 * h);
        const bool add_mu = mu_v && l_tot > 0.0f;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                mv[c][r4] = add_mu ? *reinterpret_cast<const float4*>(vslds + D + 32 * c + 8 * r4 + 4 * h)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        uint8_t* mine = stg + qi * RS;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int ch0 = 32 * c + 8 * r4 + 4 * h;
                const float4 s4 = sv[c][r4], m4 = mv[c][r4];
                const float vals[4] = {acc[c][4 * r4] * s4.x * inv_l + m4.x,
                                       acc[c][4 * r4 + 1] * s4.y * inv_l + m4.y,
                                       acc[c][4 * r4 + 2] * s4.z * inv_l + m4.z,
                                       acc[c][4 * r4 + 3] * s4.w * inv_l + m4.w};
                // (rounded to nearest even by the packed converts)
                const int byte = 2 * ch0;              // 8-byte half of granule byte / 16
                *reinterpret_cast<uint2*>(mine + ((((byte >> 4) ^ (qi % NGR)) << 4) | (byte & 15))) =
                    make_uint2(pack16<DT>(vals[0], vals[1]), pack16<DT>(vals[2], vals[3]));
            }
        if (lse && h == 0 && my_q < nq)
            lse[si.lse0 + (int64_t)w.head * P.lse_hstride + my_q] =
                l_tot > 0.0f ? (m_run + __log2f(l_tot) - (PVH ? 0.0f : LOG2_448)) * LN2 : -INFINITY;
        // whole rows: D/8 granules of 16 bytes per row, 32 rows
        uint16_t* obase = o + si.o_el + (int64_t)w.head * P.os.h;
        constexpr int GPRW = D / 8;
#pragma unroll
        for (int i = 0; i < 32 * GPRW / 64; ++i) {
            const int idx = lane + 64 * i;
            const int row = idx / GPRW, gr = idx % GPRW;
            const int q = w.q0 + row;
            const uint4 val = *reinterpret_cast<const uint4*>(stg + row * RS + ((gr ^ (row % NGR)) << 4));
            if (q < nq) *reinterpret_cast<uint4*>(obase + (int64_t)q * P.os.n + 8 * gr) = val;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode kernel (a split key range with few queries): one wave per
// workgroup and one (sequence, kv head, split) per wave.  The query heads of
// the GQA group and their queries are packed into the wave's 32 rows (row r:
// head hkv*G + r / nq, query r % nq; the host only uses it when G*nq <= 32),
// so every row of the MFMA tile is a real query.  The wave stages its own
// tiles in LDS: K(t+1) streams in under softmax(t), V(t) under Q.K(t).  The
// tiles, the online softmax and the split partials are those of k_attn, so
// the result is the same recipe.
// ---------------------------------------------------------------------------
// Wait until at most n of this wave's vector memory operations (its
// direct-to-LDS copies) are outstanding; they complete in issue order.  The
// count is an immediate of s_waitcnt, hence one case per value (a decode
// wave never has more than 48 copies in flight).
__device__ inline void wait_vm(int n) {
    switch (n) {
#define SAGE_W(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        SAGE_W(0) SAGE_W(1) SAGE_W(2) SAGE_W(3) SAGE_W(4) SAGE_W(5) SAGE_W(6) SAGE_W(7)
        SAGE_W(8) SAGE_W(9) SAGE_W(10) SAGE_W(11) SAGE_W(12) SAGE_W(13) SAGE_W(14) SAGE_W(15)
        SAGE_W(16) SAGE_W(17) SAGE_W(18) SAGE_W(19) SAGE_W(20) SAGE_W(21) SAGE_W(22) SAGE_W(23)
        SAGE_W(24) SAGE_W(25) SAGE_W(26) SAGE_W(27) SAGE_W(28) SAGE_W(29) SAGE_W(30) SAGE_W(31)
        SAGE_W(32) SAGE_W(33) SAGE_W(34) SAGE_W(35) SAGE_W(36) SAGE_W(37) SAGE_W(38) SAGE_W(39)
        SAGE_W(40) SAGE_W(41) SAGE_W(42) SAGE_W(43) SAGE_W(44) SAGE_W(45) SAGE_W(46) SAGE_W(47)
        SAGE_W(48)
#undef SAGE_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Bytes of one score-bias stage of a decode wave: G heads of 128 floats,
// copied two heads (1 KB) at a time.
__host__ __device__ constexpr int dec_ds_stage(int G) { return (G + 1) / 2 * 1024; }

// LDS bytes of one decode wave: K and V^T stages and two score-bias stages.
template <int D, bool HAS_DS, bool PVH>
__host__ __device__ constexpr int dec_lds_bytes(int G) {
    return Tile<D, PVH>::KBYTES + Tile<D, PVH>::VBYTES + (HAS_DS ? 2 * dec_ds_stage(G) : 0);
}

// Per-lane source offsets of one wave's 1 KB copies of a K tile and a V^T
// tile into the LDS images described by Tile (dense rows, swizzled slots).
// A copy spans 8 or 16 key rows (4 or 8 V^T rows), so the pattern of the key
// permutation and swizzle (32 key rows, 16 V^T rows) takes KPER (VPER)
// copies; later copies repeat it shifted by whole periods.  D = 96 copies
// only the 96 V^T rows that the P.V reads.
template <int D, bool PVH>
struct WaveDma {
    using T = Tile<D, PVH>;
    static constexpr int KCOPIES = T::KBYTES / 1024;
    static constexpr int VCOPIES = D * T::VRB / 1024;
    static constexpr int KPER = 32 * T::KRS / 1024;
    static constexpr int VPER = 16 * T::VRB / 1024;
    static_assert(KCOPIES % KPER == 0 && VCOPIES % VPER == 0, "copy periods");
    int k[KPER], v[VPER];

    __device__ inline void init(int npk) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int o = 1024 * i + 16 * lane;
            const int row = o / T::KRS, slot = (o % T::KRS) / 16;
            int lg = slot ^ swz<T::KRS>(row);
            if (D == 96 && lg >= 6) lg &= 1;       // unused slots: any in-row granule
            k[i] = key_of_row(row) * D + lg * 16;
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int o = 1024 * i + 16 * lane;
            const int ch = o / T::VRB, vslot = (o % T::VRB) / 16;
            v[i] = ch * npk * T::VES + ((vslot ^ swz<T::VRB>(ch)) << 4);
        }
    }
    __device__ inline void stage_k(uint8_t* kst, const int8_t* kbase, int t) const {
        const int8_t* kt = kbase + (int64_t)t * KVT * D;
#pragma unroll
        for (int i = 0; i < KCOPIES; ++i)
            dma16(kt + k[i % KPER] + (i / KPER) * 32 * D, kst + 1024 * i);
    }
    __device__ inline void stage_v(uint8_t* vst, const uint8_t* vbase, int npk, int t) const {
        const uint8_t* vt = vbase + t * (KVT * T::VES);
#pragma unroll
        for (int i = 0; i < VCOPIES; ++i)
            dma16(vt + v[i % VPER] + (int64_t)(i / VPER) * 16 * npk * T::VES, vst + 1024 * i);
    }
};

template <int D, int DT, bool HAS_DS, bool PVH, int QB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_decode(KParams P, const int8_t* __restrict__ qc,
                                               const float* __restrict__ qsc,
                                               const int8_t* __restrict__ kc,
                                               const float* __restrict__ ksc,
                                               const uint8_t* __restrict__ vc,
                                               const float* __restrict__ vsc,
                                               const float* __restrict__ ds,
                                               const float* __restrict__ mu_v) {
    extern __shared__ __align__(16) uint8_t smem[];
    using T = Tile<D, PVH>;
    using O = WaveDma<D, PVH>;
    int local;
    auto per = [&](int) { return P.hkv * P.nsplit; };
    const int s = find_seq(P, blockIdx.x, per, &local);
    const SeqInfo si = seq_info(P, s);
    const int split = local / P.hkv, hkv = local % P.hkv;   // kv head fastest
    const int nq = si.nq, nkv = si.nkv;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, qi = lane & 31;
    const int G = P.group;
    const bool row_ok = qi < G * nq;
    const int hl = row_ok ? qi / nq : 0, my_q = row_ok ? qi % nq : 0;
    const int head = hkv * G + hl;
    const int diag = my_q + nkv - nq;             // last visible key of the row (causal)
    const int lim = P.causal ? min(diag, nkv - 1) : nkv - 1;
    const int diag0 = nkv - nq;                   // ... of the group's first query
    const int nt_all = (nkv + KVT - 1) / KVT;
    const int t0 = split * P.kv_tiles;
    const int t1 = min(nt_all, t0 + P.kv_tiles);

    const int64_t krow0 = (si.rk * P.hkv + (int64_t)hkv * si.npk);
    const int8_t* kbase = kc + krow0 * D;
    const uint8_t* vbase = vc + krow0 * D * T::VES;
    const float* kscb = ksc + krow0 / QB;
    const float* dsb = HAS_DS ? ds + si.rk * P.hq + (int64_t)(hkv * G) * si.npk : nullptr;
    uint8_t* kbuf = smem;
    uint8_t* vbuf = smem + T::KBYTES;
    uint8_t* dsbuf = vbuf + T::VBYTES;            // two score-bias stages
    O off;
    off.init(si.npk);
    const int nds = HAS_DS ? (G + 1) / 2 : 0;     // score-bias copies per tile
    auto stage_ds = [&](int t, int which) {
        if constexpr (HAS_DS) {
            for (int i = 0; i < nds; ++i) {
                const int hs = min(2 * i + h, G - 1);
                dma16(dsb + (int64_t)hs * si.npk + t * KVT + qi * 4,
                      dsbuf + which * dec_ds_stage(G) + i * 1024);
            }
        }
    };

    v4i qf[D / 32];
    float sq = 0.0f;
    const int64_t qrow0 = si.rq * P.hq + (int64_t)head * si.npq;
    if (row_ok && t0 < t1) {
        load_q<D>(qc + (qrow0 + my_q) * D, qf);
        sq = qsc[(qrow0 + my_q) / QB];
    } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c) asm volatile("" ::"v"(qf[c]));
    asm volatile("" : "+v"(sq));

    v16f acc[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    v8i pb[2];
    v4i ph[PVH ? 8 : 1];
    v16i sacc[4];

    // vmcnt counts at most 63 operations.  When K, its bias and V of a tile
    // would exceed that (16-bit V with the bias of many heads), the wave
    // waits for K(t) and its bias before issuing V(t), and issues the bias
    // of tile t+1 only once V(t) has landed: at most V + K in flight.
    const bool early = O::KCOPIES + nds + O::VCOPIES > 60;
    if (t0 < t1) {
        off.stage_k(kbuf, kbase, t0);
        stage_ds(t0, 0);
    }
    for (int t = t0; t < t1; ++t) {
        const int r = t - t0;
        // V(t) streams in under Q.K(t) and softmax(t)
        if (early) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        off.stage_v(vbuf, vbase, si.npk, t);
        wait_vm(O::VCOPIES);                      // K(t) and its bias have landed
        qk_tile<D>(kbuf, qf, sacc);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // K(t) reads done
        int nnext = 0;
        const bool more = t + 1 < t1;
        if (more) {                               // K(t+1) streams in under the rest
            off.stage_k(kbuf, kbase, t + 1);
            if (!early) stage_ds(t + 1, (r + 1) & 1);
            nnext = O::KCOPIES + (early ? 0 : nds);
        }
        constexpr int NB = KVT / QB;
        auto cs = [&](int b) {
            const float ks = kscb[NB * t + b];
            return fmaxf(HAS_DS ? sq * ks : sq * ks * P.sml2, FLT_MIN);
        };
        const float c0 = cs(0), c1 = cs(1);
        const float c2 = NB == 4 ? cs(NB == 4 ? 2 : 0) : 0.0f;
        const float c3 = NB == 4 ? cs(NB == 4 ? 3 : 0) : 0.0f;
        const int kt0 = t * KVT + 16 * h;
        const float* dsl = HAS_DS ? reinterpret_cast<const float*>(dsbuf + (r & 1) * dec_ds_stage(G)) +
                                        hl * KVT
                                  : nullptr;
        const bool need_mask = (t + 1) * KVT > nkv || (P.causal && (t + 1) * KVT - 1 > diag0);
        float alpha;
        if (need_mask)
            alpha = softmax_tile<true, HAS_DS, PVH, DT, QB>(sacc, pb, ph, c0, c1, c2, c3, dsl,
                                                            P.sml2, kt0, lim, m_run, l_run);
        else
            alpha = softmax_tile<false, HAS_DS, PVH, DT, QB>(sacc, pb, ph, c0, c1, c2, c3, dsl,
                                                             P.sml2, kt0, lim, m_run, l_run);
        wait_vm(nnext);                           // V(t) has landed
        if (early && more) stage_ds(t + 1, (r + 1) & 1);
        rescale<D>(acc, alpha);
        if constexpr (PVH) pv_tile_h<D, DT>(vbuf, ph, acc);
        else pv_tile<D>(vbuf, pb, acc);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // V(t) reads done
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // this split's partial of each row (as in k_attn's split epilogue)
    const float l_tot = swap_sum(l_run);
    if (row_ok) {
        const int64_t row = si.lse0 + (int64_t)head * P.lse_hstride + my_q;
        const int64_t pr = (int64_t)split * P.rows_total + row;
        const int64_t vsb = ((int64_t)si.sid * P.hkv + hkv) * D;
        const bool add_mu = mu_v && l_tot > 0.0f;
        float* po = P.part_o + pr * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int ch0 = 32 * c + 8 * r4 + 4 * h;
                const float4 s4 = PVH ? make_float4(1.f, 1.f, 1.f, 1.f)
                                      : *reinterpret_cast<const float4*>(vsc + vsb + ch0);
                const float4 m4 = add_mu ? *reinterpret_cast<const float4*>(mu_v + vsb + ch0)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4*>(po + ch0) =
                    make_float4(fmaf(acc[c][4 * r4], s4.x, m4.x * l_tot),
                                fmaf(acc[c][4 * r4 + 1], s4.y, m4.y * l_tot),
                                fmaf(acc[c][4 * r4 + 2], s4.z, m4.z * l_tot),
                                fmaf(acc[c][4 * r4 + 3], s4.w, m4.w * l_tot));
            }
        if (h == 0) *reinterpret_cast<float2*>(P.part_ml + 2 * pr) = make_float2(m_run, l_tot);
    }
}

// ---------------------------------------------------------------------------
// Test export of the E4M3 conversion: thread i converts the FP32 bit patterns
// first + 4i .. first + 4i + 3 and packs them into one word exactly as the
// fused kernel packs its P operand (low half, then high half).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(WG) void k_e4m3_dump(uint32_t first, uint32_t count,
                                                  uint8_t* __restrict__ out) {
    const uint32_t i = blockIdx.x * WG + threadIdx.x;
    const uint32_t e0 = 4u * i;
    if (e0 >= count) return;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(first + e0 + k);
    uint32_t u = e4m3_pk<false>(x[0], x[1], __float_as_uint(x[0]));
    u = e4m3_pk<true>(x[2], x[3], u);
    if (e0 + 4 <= count) {
        *reinterpret_cast<uint32_t*>(out + e0) = u;
    } else {
        for (uint32_t k = 0; e0 + k < count; ++k) out[e0 + k] = (uint8_t)(u >> (8 * k));
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {

int wg_count_host(const KParams& P, int waves) {
    const int hpw = heads_per_wg(P.group);
    const int rows = 32 * waves / hpw;
    const int per_nq = P.hkv * (P.group / hpw);
    if (P.tab.uniform) return P.tab.n * per_nq * ((P.tab.nq[0] + rows - 1) / rows);
    int tot = 0;
    for (int s = 0; s < P.tab.n; ++s) tot += per_nq * ((P.tab.nq[s] + rows - 1) / rows);
    return tot;
}


// Allow a kernel its dynamic LDS beyond the default, once per device (the
// attribute belongs to the function on the current device).  `done` holds one
// bit per device id below 64; devices above that set it on every call.  Two
// threads racing on a device both set it, which is harmless.
hipError_t lds_attr(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t{1} << dev) : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_relaxed);
    return hipSuccess;
}

template <int D, int DT, bool HAS_DS, bool PVH, int QB, bool BQS = false>
hipError_t attn_d(const KParams& P, const int8_t* qc, const float* qsc, const int8_t* kc,
                  const float* ksc, const uint8_t* vc, const float* vsc, const float* ds,
                  const float* mu_v, void* o, float* lse, const int8_t* mcode, const float* mcs,
                  hipStream_t st) {
    static std::atomic<uint64_t> attr_set{0};
    // (+64 bytes: the absmax slots of the kernel's own Q quantization; then
    // the V scales and means of the epilogue, 2*D floats)
    constexpr int LDS = lds_bytes<D, HAS_DS, PVH, BQS, QB>() + 64 + 8 * D;
    auto* kern = &k_attn<D, DT, HAS_DS, PVH, QB, false, BQS>;
    hipError_t e = lds_attr(reinterpret_cast<const void*>(kern), LDS, attr_set);
    if (e != hipSuccess) return e;
    const int nblocks = wg_count_host(P, FWD_WAVES) * P.nsplit;
    if (nblocks <= 0) return hipSuccess;
    kern<<<nblocks, FWD_NT, LDS, st>>>(P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v,
                                       static_cast<uint16_t*>(o), lse, mcode, mcs);
    return hipGetLastError();
}

template <int D, int DT, bool HAS_DS, bool PVH, int QB>
hipError_t decode_d(const KParams& P, const int8_t* qc, const float* qsc, const int8_t* kc,
                    const float* ksc, const uint8_t* vc, const float* vsc, const float* ds,
                    const float* mu_v, hipStream_t st) {
    static std::atomic<uint64_t> attr_set{0};
    hipError_t e = lds_attr(reinterpret_cast<const void*>(&k_decode<D, DT, HAS_DS, PVH, QB>),
                            dec_lds_bytes<D, HAS_DS, PVH>(32), attr_set);
    if (e != hipSuccess) return e;
    const int nblocks = P.tab.n * P.hkv * P.nsplit;
    if (nblocks <= 0) return hipSuccess;
    k_decode<D, DT, HAS_DS, PVH, QB><<<nblocks, 64, dec_lds_bytes<D, HAS_DS, PVH>(P.group), st>>>(
        P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v);
    return hipGetLastError();
}

}  // namespace

int decode_waves_per_cu(int d, bool pv_half, bool has_ds, int group) {
    int b;
#define SAGE_DL(D)                                                                        \
    b = pv_half ? (has_ds ? dec_lds_bytes<D, true, true>(group) : dec_lds_bytes<D, false, true>(group)) \
                : (has_ds ? dec_lds_bytes<D, true, false>(group) : dec_lds_bytes<D, false, false>(group))
    if (d == 64) SAGE_DL(64);
    else if (d == 96) SAGE_DL(96);
    else SAGE_DL(128);
#undef SAGE_DL
    return std::max(1, std::min(4, LDS_PER_CU / b));
}

bool use_decode_kernel(const KParams& P) {
    if (P.kv_tiles <= 0 || P.bqs) return false;
    int mq = 0;
    const int n = P.tab.uniform ? 1 : P.tab.n;
    for (int s = 0; s < n; ++s) mq = std::max(mq, P.tab.nq[s]);
    return P.group * std::max(mq, 1) <= DEC_ROWS;
}

hipError_t launch_attn(const KParams& P, int dtype, const int8_t* qc, const float* qsc,
                       const int8_t* kc, const float* ksc, const uint8_t* vc, const float* vsc,
                       const float* ds, const float* mu_v, void* o, float* lse,
                       const int8_t* mcode, const float* mcs, hipStream_t st) {
    const bool dec = use_decode_kernel(P);
    if (P.bqs && (!ds || !mcode || !mcs || P.pv_half)) return hipErrorInvalidValue;
#define SAGE_AQ(D, DT, PVH, QB)                                                                  \
    do {                                                                                         \
        if (dec)                                                                                 \
            return ds ? decode_d<D, DT, true, PVH, QB>(P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v, st) \
                      : decode_d<D, DT, false, PVH, QB>(P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v, st); \
        if constexpr (!PVH)                                                                      \
            if (P.bqs)                                                                           \
                return attn_d<D, DT, true, false, QB, true>(P, qc, qsc, kc, ksc, vc, vsc, ds,   \
                                                            mu_v, o, lse, mcode, mcs, st);      \
        return ds ? attn_d<D, DT, true, PVH, QB>(P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v, o, lse, \
                                                 nullptr, nullptr, st)                           \
                  : attn_d<D, DT, false, PVH, QB>(P, qc, qsc, kc, ksc, vc, vsc, ds, mu_v, o, lse,\
                                                  nullptr, nullptr, st);                         \
    } while (0)
#define SAGE_AH(D, DT, PVH)                    \
    do {                                       \
        if (P.qb == 32) SAGE_AQ(D, DT, PVH, 32); \
        SAGE_AQ(D, DT, PVH, QBLK);             \
    } while (0)
#define SAGE_A(D, DT)                   \
    do {                                \
        if (P.pv_half) SAGE_AH(D, DT, true); \
        SAGE_AH(D, DT, false);          \
    } while (0)
    if (dtype == 0) {
        if (P.d == 64) { SAGE_A(64, 0); }
        if (P.d == 96) { SAGE_A(96, 0); }
        SAGE_A(128, 0);
    } else {
        if (P.d == 64) { SAGE_A(64, 1); }
        if (P.d == 96) { SAGE_A(96, 1); }
        SAGE_A(128, 1);
    }
#undef SAGE_A
#undef SAGE_AH
#undef SAGE_AQ
}

namespace {
template <int D>
hipError_t qk_dump_d(const KParams& P, const int8_t* qc, const int8_t* kc, int32_t* s_out,
                     hipStream_t st) {
    static std::atomic<uint64_t> attr_set{0};
    auto* kern = &k_attn<D, 0, false, false, QBLK, true>;
    hipError_t e = lds_attr(reinterpret_cast<const void*>(kern), lds_bytes<D, false, false>(),
                            attr_set);
    if (e != hipSuccess) return e;
    const int nblocks = wg_count_host(P, FWD_WAVES);
    if (nblocks <= 0) return hipSuccess;
    kern<<<nblocks, FWD_NT, lds_bytes<D, false, false>(), st>>>(
        P, qc, nullptr, kc, nullptr, nullptr, nullptr, nullptr, nullptr,
        reinterpret_cast<uint16_t*>(s_out), nullptr, nullptr, nullptr);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_qk_dump(const KParams& P, const int8_t* qc, const int8_t* kc, int32_t* s_out,
                          hipStream_t st) {
    if (P.d == 64) return qk_dump_d<64>(P, qc, kc, s_out, st);
    if (P.d == 96) return qk_dump_d<96>(P, qc, kc, s_out, st);
    return qk_dump_d<128>(P, qc, kc, s_out, st);
}


// ---------------------------------------------------------------------------
// Merge of a split key range (flash-decoding): per row, M = max m_s,
// w_s = 2^(m_s - M), L = sum w_s l_s, o = sum w_s part_s / L, the partials
// already holding acc*v_scale + mu_v*l.  One wave per row: lane j first takes
// the (m, l) of splits j, j+64, ..., then the wave walks the splits in order
// with each lane accumulating two channels (coalesced 8-byte reads of every
// partial row).  Every split writes its partial (zeros and m = -inf when it
// saw no key), so the loads need no guard.
// ---------------------------------------------------------------------------
__device__ inline float wave_sum64(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <int DT>
__global__ __launch_bounds__(256) void k_merge(MergeArgs M) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M.rows_total) return;             // the whole wave leaves
    const int64_t rs = M.rows_total;
    float mx = -INFINITY;
    for (int s0 = 0; s0 < M.nsplit; s0 += 64)
        if (s0 + lane < M.nsplit) mx = fmaxf(mx, M.part_ml[2 * ((s0 + lane) * rs + row)]);
    mx = wave_max64(mx);
    const int c0 = 2 * lane;
    const bool act = c0 < M.d;
    float lp = 0.0f, a0 = 0.0f, a1 = 0.0f;
    if (mx != -INFINITY) {
        for (int s0 = 0; s0 < M.nsplit; s0 += 64) {
            float wl = 0.0f;
            if (s0 + lane < M.nsplit) {
                const float2 ml = *reinterpret_cast<const float2*>(M.part_ml + 2 * ((s0 + lane) * rs + row));
                wl = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml.x - mx);
                lp = fmaf(wl, ml.y, lp);
            }
            const int cnt = min(64, M.nsplit - s0);
            const float* po = M.part_o + ((int64_t)s0 * rs + row) * M.d + c0;
            const int64_t step = rs * M.d;
            int j = 0;
            for (; j + 4 <= cnt; j += 4) {
                float2 p[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    p[u] = act ? *reinterpret_cast<const float2*>(po + (j + u) * step)
                               : make_float2(0.f, 0.f);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float w = __shfl(wl, j + u);
                    a0 = fmaf(w, p[u].x, a0);
                    a1 = fmaf(w, p[u].y, a1);
                }
            }
            for (; j < cnt; ++j) {
                const float2 p = act ? *reinterpret_cast<const float2*>(po + j * step)
                                     : make_float2(0.f, 0.f);
                const float w = __shfl(wl, j);
                a0 = fmaf(w, p.x, a0);
                a1 = fmaf(w, p.y, a1);
            }
        }
    }
    const float L = wave_sum64(lp);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    int64_t off;
    if (M.varlen) {
        const int64_t h = row / M.total_q, tok = row % M.total_q;
        off = tok * M.os.n + h * M.os.h;
    } else {
        const int64_t per_seq = (int64_t)M.hq * M.nq;
        const int64_t sidx = row / per_seq, rem = row % per_seq;
        off = sidx * M.os.b + (rem / M.nq) * M.os.h + (rem % M.nq) * M.os.n;
    }
    if (act)
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(M.o) + off + c0) =
            f2h_bits<DT>(a0 * inv) | (f2h_bits<DT>(a1 * inv) << 16);
    if (lane == 0 && M.lse)
        M.lse[row] = L > 0.0f ? (mx + __log2f(L) - M.poff) * LN2 : -INFINITY;
}

int attn_base_wgs(const KParams& P) { return wg_count_host(P, FWD_WAVES); }

hipError_t launch_merge(const MergeArgs& M, int dtype, hipStream_t st) {
    if (M.rows_total <= 0) return hipSuccess;
    const int64_t nb = (M.rows_total + 3) / 4;   // four rows (waves) per workgroup
    if (dtype == 0) k_merge<0><<<(unsigned)nb, 256, 0, st>>>(M);
    else k_merge<1><<<(unsigned)nb, 256, 0, st>>>(M);
    return hipGetLastError();
}

hipError_t launch_e4m3_dump(uint32_t first, uint32_t count, uint8_t* out, hipStream_t st) {
    if (count == 0) return hipSuccess;
    const uint32_t threads = (count + 3) / 4;
    const uint32_t blocks = (threads + WG - 1) / WG;
    k_e4m3_dump<<<blocks, WG, 0, st>>>(first, count, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The workspace of the allocation-free entry point: a file-scope device array
// (each device the library runs on holds its own copy until the process
// ends).  In host code `scratch` only stands for the symbol: its device
// address on a device comes from hipGetSymbolAddress with that device
// current, taken once per device and kept; only that address is passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[NOALLOC_WS_MAX];

hipError_t noalloc_workspace(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::vector<void*> addr;     // per device id; nullptr until taken
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace sage
