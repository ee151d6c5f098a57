// abi_drive.cpp -- drives the host side of the libsage C ABI (include/sage.h)
// through its size queries and entry points with valid and invalid
// descriptors, cu_seqlens tables (empty, ragged, more sequences than one
// launch table, non-monotone), flags and pointers, so that a build with the
// host AddressSanitizer / UndefinedBehaviorSanitizer can check the argument
// checks, the workspace plan and the sequence tables.  Pointers are fake and
// never dereferenced: every call fails a host check, or the device check,
// before any work is launched.  Test infrastructure: built with
// launch_stubs.cpp by tests/test_sanitizers.py; exits non-zero on an
// unexpected status.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "sage.h"

static int fails = 0;
#define EXPECT(call, want)                                                                \
    do {                                                                                  \
        const sage_status st_ = (call);                                                   \
        if (st_ != (want)) {                                                              \
            std::fprintf(stderr, "line %d: %s gave %d (%s), expected %d\n", __LINE__, #call, \
                         (int)st_, sage_status_string(st_), (int)(want));                 \
            ++fails;                                                                      \
        }                                                                                 \
    } while (0)
// a valid call stops at the device check (no GPU) or at the first launch
#define EXPECT_REACHES_DEVICE(call)                                                       \
    do {                                                                                  \
        const sage_status st_ = (call);                                                   \
        if (st_ != SAGE_ERR_HIP && st_ != SAGE_ERR_ARCH && st_ != SAGE_OK) {              \
            std::fprintf(stderr, "line %d: %s gave %d (%s)\n", __LINE__, #call, (int)st_,  \
                         sage_status_string(st_));                                        \
            ++fails;                                                                      \
        }                                                                                 \
    } while (0)

static void* fake(uintptr_t a = 0x10000) { return reinterpret_cast<void*>(a); }

static sage_quant_bufs fake_bufs() {
    sage_quant_bufs b{};
    auto f = [](uintptr_t a) { return reinterpret_cast<float*>(a); };
    b.mu_q = f(0x10000); b.mu_k = f(0x20000); b.mu_v = f(0x30000);
    b.q_codes = reinterpret_cast<int8_t*>(0x40000); b.q_scale = f(0x50000);
    b.k_codes = reinterpret_cast<int8_t*>(0x60000); b.k_scale = f(0x70000);
    b.v_codes = reinterpret_cast<uint8_t*>(0x80000); b.v_scale = f(0x90000);
    b.delta_s = f(0xa0000); b.mu_qb = f(0xb0000);
    b.mu_q_code = reinterpret_cast<int8_t*>(0xc0000); b.mu_q_cscale = f(0xd0000);
    return b;
}

static void dense_cases() {
    const int dims[] = {64, 96, 128};
    for (int d : dims)
        for (int sq = 0; sq <= 2; ++sq)
            for (int pv = 0; pv <= 1; ++pv)
                for (int qb : {0, 32, 64})
                    for (int split : {0, 256, SAGE_KV_SPLIT_AUTO}) {
                        sage_attn_desc desc;
                        sage_desc_init(&desc, d == 96 ? SAGE_BF16 : SAGE_F16,
                                       d == 128 ? SAGE_HND : SAGE_NHD, 2, 8, 2, 1 + d, 300 + d, d);
                        desc.smooth_q = sq;
                        desc.smooth_v = pv;
                        desc.pv_mode = pv;
                        desc.qk_block = qb;
                        desc.kv_split = split;
                        desc.is_causal = (d / 32) & 1;
                        const bool bad = sq == 2 && pv == 1;
                        sage_quant_sizes z;
                        size_t ws = 0;
                        int32_t keys = 0;
                        EXPECT(sage_quant_buf_sizes(&desc, nullptr, nullptr, 0, &z),
                               bad ? SAGE_ERR_FLAGS : SAGE_OK);
                        EXPECT(sage_workspace_size(&desc, nullptr, nullptr, 0, &ws),
                               bad ? SAGE_ERR_FLAGS : SAGE_OK);
                        EXPECT(sage_kv_split_size(&desc, nullptr, nullptr, 0, &keys),
                               bad ? SAGE_ERR_FLAGS : SAGE_OK);
                        if (bad) continue;
                        EXPECT_REACHES_DEVICE(sage_attn_fwd(&desc, fake(), fake(), fake(), fake(),
                                                            nullptr, fake(), ws + 4096, nullptr));
                        sage_quant_bufs b = fake_bufs();
                        EXPECT_REACHES_DEVICE(sage_quant_qkv(&desc, fake(), fake(), fake(), nullptr,
                                                             nullptr, 0, &b, fake(), ws + 4096,
                                                             nullptr));
                        EXPECT_REACHES_DEVICE(sage_attn_fwd_quantized(&desc, nullptr, nullptr, 0, &b,
                                                                      fake(), nullptr, fake(),
                                                                      ws + 4096, nullptr));
                        EXPECT(sage_attn_fwd(&desc, fake(), fake(), fake(), fake(), nullptr, fake(),
                                             0, nullptr),
                               SAGE_ERR_WORKSPACE);
                        EXPECT(sage_attn_fwd(&desc, fake(0x10008), fake(), fake(), fake(), nullptr,
                                             fake(), ws + 4096, nullptr),
                               SAGE_ERR_ALIGN);
                        EXPECT(sage_attn_fwd(&desc, nullptr, fake(), fake(), fake(), nullptr,
                                             fake(), ws + 4096, nullptr),
                               SAGE_ERR_NULL);
                    }
}

static void varlen_cases() {
    sage_attn_desc desc;
    sage_desc_init(&desc, SAGE_F16, SAGE_NHD, 0, 4, 2, 0, 0, 128);
    desc.smooth_q = 2;
    // empty sequences, ragged lengths, and 40 sequences (two launch tables)
    std::vector<std::vector<int32_t>> lens = {
        {0}, {5, 0, 70, 33}, {0, 0, 0}, {1},
    };
    std::vector<int32_t> many;
    for (int i = 0; i < 40; ++i) many.push_back((i * 37) % 150);
    lens.push_back(many);
    for (const auto& lq : lens) {
        const int n = (int)lq.size();
        std::vector<int32_t> cq(n + 1, 0), ck(n + 1, 0);
        for (int i = 0; i < n; ++i) {
            cq[i + 1] = cq[i] + lq[i];
            ck[i + 1] = ck[i] + (lq[i] * 7) % 300 + (i & 1);
        }
        for (int sq = 0; sq <= 2; ++sq)
            for (int split : {0, SAGE_KV_SPLIT_AUTO}) {
                desc.smooth_q = sq;
                desc.kv_split = split;
                sage_quant_sizes z;
                size_t ws = 0;
                int32_t keys = 0;
                EXPECT(sage_quant_buf_sizes(&desc, cq.data(), ck.data(), n, &z), SAGE_OK);
                EXPECT(sage_workspace_size(&desc, cq.data(), ck.data(), n, &ws), SAGE_OK);
                EXPECT(sage_kv_split_size(&desc, cq.data(), ck.data(), n, &keys), SAGE_OK);
                EXPECT_REACHES_DEVICE(sage_attn_fwd_varlen(&desc, cq.data(), ck.data(), n, fake(),
                                                           fake(), fake(), fake(), nullptr, fake(),
                                                           ws + 4096, nullptr));
                sage_quant_bufs b = fake_bufs();
                EXPECT_REACHES_DEVICE(sage_debug_qk_int32(&desc, cq.data(), ck.data(), n, &b,
                                                          reinterpret_cast<int32_t*>(fake()),
                                                          nullptr));
            }
    }
    // a table that is not a prefix sum from 0, or that decreases
    std::vector<int32_t> bad1 = {1, 5, 9}, bad2 = {0, 9, 5}, good = {0, 4, 8};
    EXPECT(sage_workspace_size(&desc, bad1.data(), good.data(), 2, nullptr), SAGE_ERR_NULL);
    size_t ws;
    EXPECT(sage_workspace_size(&desc, bad1.data(), good.data(), 2, &ws), SAGE_ERR_SEQLENS);
    EXPECT(sage_workspace_size(&desc, bad2.data(), good.data(), 2, &ws), SAGE_ERR_SEQLENS);
    EXPECT(sage_workspace_size(&desc, good.data(), bad2.data(), 2, &ws), SAGE_ERR_SEQLENS);
    EXPECT(sage_workspace_size(&desc, good.data(), good.data(), -1, &ws), SAGE_ERR_SHAPE);
}

static void invalid_descriptors() {
    size_t ws;
    EXPECT(sage_workspace_size(nullptr, nullptr, nullptr, 0, &ws), SAGE_ERR_NULL);
    sage_attn_desc d;
    auto reset = [&]() { sage_desc_init(&d, SAGE_F16, SAGE_HND, 2, 8, 2, 100, 300, 128); };
    reset(); d.dtype = 7; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_DTYPE);
    reset(); d.layout = 5; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_LAYOUT);
    reset(); d.head_dim = 80; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_HEAD_DIM);
    reset(); d.hq = 7; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_GQA);
    reset(); d.nq = -1; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_SHAPE);
    reset(); d.nkv = (1 << 24) + 1; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_SHAPE);
    reset(); d.q_stride[1] = 3; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_STRIDE);
    reset(); d.smooth_q = 3; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_FLAGS);
    reset(); d.kv_split = 100; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_FLAGS);
    reset(); d.qk_block = 16; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_FLAGS);
    reset(); d.sm_scale = 1.0f / 0.0f; EXPECT(sage_workspace_size(&d, nullptr, nullptr, 0, &ws), SAGE_ERR_FLAGS);
    reset(); d.batch = 0;   // an empty problem is valid (after the device check) and launches nothing
    EXPECT_REACHES_DEVICE(sage_attn_fwd(&d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr));
    reset(); d.nq = 4096; d.nkv = 4096; d.hq = d.hkv = 32;   // beyond the static workspace
    EXPECT(sage_attn_fwd_noalloc(&d, fake(), fake(), fake(), fake(), nullptr, nullptr),
           SAGE_ERR_WORKSPACE);
    EXPECT(sage_debug_e4m3_encode(0, 16, nullptr, nullptr), SAGE_ERR_NULL);
    EXPECT(sage_debug_e4m3_encode(0xFFFFFFF0u, 32, reinterpret_cast<uint8_t*>(fake()), nullptr),
           SAGE_ERR_SHAPE);
    double r;
    EXPECT(sage_micro_rate(9, 16, &r, nullptr), SAGE_ERR_FLAGS);
    EXPECT(sage_micro_rate(0, 0, &r, nullptr), SAGE_ERR_SHAPE);
    for (int s = -1; s < 20; ++s) (void)sage_status_string(s);
    (void)sage_status_string(999);
    if (sage_abi_version() != SAGE_ABI_VERSION) ++fails;
}

int main() {
    dense_cases();
    varlen_cases();
    invalid_descriptors();
    if (fails) {
        std::fprintf(stderr, "%d unexpected statuses\n", fails);
        return 1;
    }
    std::printf("abi drive: ok\n");
    return 0;
}
