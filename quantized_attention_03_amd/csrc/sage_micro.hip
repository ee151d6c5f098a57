// sage_micro.hip -- micro-benchmarks of the execution units the fused kernel
// depends on: the dense INT8 and FP8 matrix instructions of the two products
// (Q.K^T in INT8, P.V in FP8: ComfyUI blog on SageAttention, feature item 2)
// and the VALU rates of the softmax (v_exp_f32, v_fma_f32).  Each runs
// independent dependency chains in 512-thread workgroups, four per compute
// unit (as many waves per SIMD as the registers allow), so that a measured
// rate can be set beside the part's published peak.
#include "sage_internal.h"

namespace sage {

// Written only when a result equals a value no chain reaches, so that the
// chains are kept but nothing is stored in practice (external linkage keeps
// the compiler from dropping the store and, with it, the chains).
__device__ float g_micro_sink[64];

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int MICRO_NT = 512;   // threads per workgroup
constexpr int MICRO_WG_PER_CU = 4;
constexpr int CHAINS = 4;       // independent accumulators per wave (matrix ops)
constexpr int VCHAINS = 8;      // independent registers per lane (VALU ops)

template <int OP>
__global__ __launch_bounds__(MICRO_NT) void k_micro(int reps) {
    const int lane = threadIdx.x & 63;
    float s = 0.0f;
    if constexpr (OP == MICRO_I8) {
        const v4i a = {lane, 1, 2, 3}, b = {3, 2, 1, lane};
        v16i c[CHAINS];
#pragma unroll
        for (int k = 0; k < CHAINS; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[k][r] = r + k;
        for (int it = 0; it < reps; ++it) {
#pragma unroll
            for (int k = 0; k < CHAINS; ++k)
                c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < CHAINS; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += (float)c[k][r];
    } else if constexpr (OP == MICRO_F8) {
        // E4M3 codes 0x38 (1.0) and 0x30 (0.5) in every byte
        const v8i a = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, lane};
        const v8i b = {0x30303030, 0x30303030, 0x30303030, 0x30303030,
                       0x30303030, 0x30303030, 0x30303030, 0x30303030};
        v16f c[CHAINS];
#pragma unroll
        for (int k = 0; k < CHAINS; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[k][r] = 0.0f;
        for (int it = 0; it < reps; ++it) {
#pragma unroll
            for (int k = 0; k < CHAINS; ++k)
                c[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[k], 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < CHAINS; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += c[k][r];
    } else {
        float x[VCHAINS];
#pragma unroll
        for (int i = 0; i < VCHAINS; ++i) x[i] = lane * 1e-3f + 0.125f * i;
        for (int it = 0; it < reps; ++it) {
#pragma unroll
            for (int i = 0; i < VCHAINS; ++i) {
                if constexpr (OP == MICRO_EXP)
                    x[i] = __builtin_amdgcn_exp2f(-x[i]);       // converges to about 0.64
                else
                    x[i] = fmaf(x[i], 0.999f, 1e-3f);          // converges to 1
            }
        }
#pragma unroll
        for (int i = 0; i < VCHAINS; ++i) s += x[i];
    }
    if (s == -1.0f) g_micro_sink[lane] = s;
}

// Operations one launch performs: 2*M*N*K per matrix instruction, one exp2
// result or two flops per lane and VALU instruction.
double micro_ops(int op, int grid, int reps) {
    const double waves = (double)grid * (MICRO_NT / 64) * reps;
    switch (op) {
        case MICRO_I8: return waves * CHAINS * 2.0 * 32 * 32 * 32;
        case MICRO_F8: return waves * CHAINS * 2.0 * 32 * 32 * 64;
        case MICRO_EXP: return waves * VCHAINS * 64.0;
        default: return waves * VCHAINS * 64.0 * 2.0;
    }
}

}  // namespace

hipError_t micro_rate(int op, int reps, double* per_s, hipStream_t st) {
    const int grid = NUM_CU * MICRO_WG_PER_CU;
    auto launch = [&]() {
        switch (op) {
            case MICRO_I8: k_micro<MICRO_I8><<<grid, MICRO_NT, 0, st>>>(reps); break;
            case MICRO_F8: k_micro<MICRO_F8><<<grid, MICRO_NT, 0, st>>>(reps); break;
            case MICRO_EXP: k_micro<MICRO_EXP><<<grid, MICRO_NT, 0, st>>>(reps); break;
            default: k_micro<MICRO_FMA><<<grid, MICRO_NT, 0, st>>>(reps); break;
        }
        return hipGetLastError();
    };
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e == hipSuccess) e = launch();                       // warm-up
    if (e == hipSuccess) e = hipEventRecord(a, st);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(b, st);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess) *per_s = ms > 0.0f ? micro_ops(op, grid, reps) / (ms * 1e-3) : 0.0;
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    return e;
}

}  // namespace sage
