// sage_api.cpp -- host side of libsage: argument checks, workspace plan,
// sequence tables and the launch sequence of the pre-pass and the fused
// kernel.  The C ABI is declared (and documented) in include/sage.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "sage.h"
#include "sage_internal.h"

using namespace sage;

namespace {

constexpr size_t ALIGN = 256;
inline size_t al(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Everything the host derives from a descriptor (and cu_seqlens).
struct Plan {
    int S = 0;
    bool varlen = false;
    int d = 0, hq = 0, hkv = 0, group = 1;
    std::vector<int32_t> nq, nkv, tq, tk;
    std::vector<int64_t> rq, rk;      // padded row bases per sequence
    int64_t rows_q = 0, rows_k = 0;   // sum of padded lengths
    int64_t total_q = 0;              // packed query tokens (varlen) for lse
    Strides qs{}, ks{}, vs{}, os{};
    float sm_scale = 0.0f;
    bool causal = false, smooth_q = false, smooth_k = false, smooth_v = false;
    bool smooth_q_blk = false;        // one Q mean per quantization block (smooth_q = 2)
    bool pv_half = false;             // 16-bit P.V operands (SAGE_PV_HALF)
    int32_t kv_split_req = 0;         // descriptor's kv_split (-1 auto, 0 none, keys)
    int32_t kv_split = 0;             // effective keys per split (0: no split)
    int32_t nsplit = 1;               // splits of the longest key range
    int64_t rows_total = 0;           // lse rows: B*hq*nq, or hq*total_q (varlen)
    int32_t max_nkv = 0;
    int32_t qb = QBLK;                // tokens per Q/K quantization block (64 or 32)
};

// Byte offsets of everything placed in a workspace (quantized tensors first,
// then scratch).  `quant_in_ws` = false gives the scratch-only layout used by
// sage_quant_qkv (whose quantized tensors are caller buffers).
struct WsLayout {
    size_t mu_q, mu_k, mu_v, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, delta_s;
    size_t mu_qb, mu_q_code, mu_q_cscale;
    size_t part_q, part_k, part_v, part_vmax, v_amax;
    size_t split_o, split_ml;         // partials of a split key range
    size_t total;
};

size_t split_o_bytes(const Plan& p) {
    return p.kv_split ? (size_t)p.nsplit * p.rows_total * p.d * 4 : 0;
}
size_t split_ml_bytes(const Plan& p) {
    return p.kv_split ? (size_t)p.nsplit * p.rows_total * 8 : 0;
}

sage_quant_sizes quant_sizes(const Plan& p) {
    sage_quant_sizes z{};
    const size_t S = p.S, d = p.d;
    z.mu_q = p.smooth_q ? S * p.hq * d * 4 : 0;
    z.mu_k = p.smooth_k ? S * p.hkv * d * 4 : 0;
    z.mu_v = p.smooth_v ? S * p.hkv * d * 4 : 0;
    z.q_codes = (size_t)p.rows_q * p.hq * d;
    z.q_scale = (size_t)p.rows_q * p.hq / p.qb * 4;
    z.k_codes = (size_t)p.rows_k * p.hkv * d;
    z.k_scale = (size_t)p.rows_k * p.hkv / p.qb * 4;
    z.v_codes = (size_t)p.rows_k * p.hkv * d * (p.pv_half ? 2 : 1);
    z.v_scale = p.pv_half ? 0 : S * p.hkv * d * 4;
    z.delta_s = p.smooth_q ? (size_t)p.rows_k * p.hq * 4 : 0;
    const size_t nqb = p.smooth_q_blk ? (size_t)p.rows_q * p.hq / p.qb : 0;
    z.mu_qb = nqb * d * 4;
    z.mu_q_code = nqb * 2 * d;
    z.mu_q_cscale = nqb * 4;
    return z;
}

WsLayout ws_layout(const Plan& p, bool quant_in_ws) {
    WsLayout w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    if (quant_in_ws) {
        const sage_quant_sizes z = quant_sizes(p);
        w.mu_q = take(z.mu_q);
        w.mu_k = take(z.mu_k);
        w.mu_v = take(z.mu_v);
        w.q_codes = take(z.q_codes);
        w.q_scale = take(z.q_scale);
        w.k_codes = take(z.k_codes);
        w.k_scale = take(z.k_scale);
        w.v_codes = take(z.v_codes);
        w.v_scale = take(z.v_scale);
        w.delta_s = take(z.delta_s);
        w.mu_qb = take(z.mu_qb);
        w.mu_q_code = take(z.mu_q_code);
        w.mu_q_cscale = take(z.mu_q_cscale);
    }
    const size_t d = p.d;
    w.part_q = take(p.smooth_q ? (size_t)p.rows_q / QBLK * p.hq * d * 4 : 0);
    w.part_k = take(p.smooth_k ? (size_t)p.rows_k / QBLK * p.hkv * d * 4 : 0);
    w.part_v = take(p.smooth_v ? (size_t)p.rows_k / QBLK * p.hkv * d * 4 : 0);
    w.part_vmax = take(p.pv_half ? 0 : (size_t)p.rows_k / QBLK * p.hkv * d * 4);
    w.v_amax = take(p.pv_half ? 0 : (size_t)p.S * p.hkv * d * 4);
    w.split_o = take(split_o_bytes(p));
    w.split_ml = take(split_ml_bytes(p));
    w.total = off + ALIGN;   // slack so that an unaligned base can be rounded up
    return w;
}

// Workspace of the fused kernel alone (sage_attn_fwd_quantized): only the
// partials of a split key range.
WsLayout ws_layout_fused(const Plan& p) {
    WsLayout w{};
    w.split_o = 0;
    w.split_ml = al(split_o_bytes(p));
    w.total = p.kv_split ? w.split_ml + al(split_ml_bytes(p)) + ALIGN : 0;
    return w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void resolve_split(Plan* p);   // below, after make_params

bool flag_ok(int32_t f) { return f == 0 || f == 1; }

// Checks on the descriptor and cu_seqlens (host only, no HIP call).
sage_status make_plan(const sage_attn_desc* desc, const int32_t* cuq, const int32_t* cuk,
                      int32_t nseq, bool varlen, Plan* out) {
    if (!desc) return SAGE_ERR_NULL;
    if (varlen && (!cuq || !cuk)) return SAGE_ERR_NULL;
    const sage_attn_desc& D = *desc;
    if (D.dtype != SAGE_F16 && D.dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
    if (D.layout != SAGE_HND && D.layout != SAGE_NHD) return SAGE_ERR_LAYOUT;
    if (!flag_ok(D.is_causal) || !(flag_ok(D.smooth_q) || D.smooth_q == SAGE_SMOOTH_Q_BLOCK) ||
        !flag_ok(D.smooth_k) ||
        !flag_ok(D.smooth_v) || (D.pv_mode != SAGE_PV_FP8 && D.pv_mode != SAGE_PV_HALF) ||
        !(D.kv_split == SAGE_KV_SPLIT_AUTO || D.kv_split == 0 ||
          (D.kv_split > 0 && D.kv_split % SAGE_KV_TILE == 0 && D.kv_split <= (1 << 24))) ||
        !(D.qk_block == 0 || D.qk_block == 64 || D.qk_block == 32) ||
        !std::isfinite(D.sm_scale) ||
        (D.smooth_q == SAGE_SMOOTH_Q_BLOCK && D.pv_mode != SAGE_PV_FP8))
        return SAGE_ERR_FLAGS;
    if (D.head_dim != 64 && D.head_dim != 96 && D.head_dim != 128) return SAGE_ERR_HEAD_DIM;
    if (D.hq < 1 || D.hkv < 1 || D.hq > 65536 || D.hkv > 65536) return SAGE_ERR_SHAPE;
    if (!varlen && (D.batch < 0 || D.nq < 0 || D.nkv < 0 || D.nq > (1 << 24) ||
                    D.nkv > (1 << 24) || D.batch > (1 << 20)))
        return SAGE_ERR_SHAPE;
    if (varlen && (nseq < 0 || nseq > (1 << 20))) return SAGE_ERR_SHAPE;
    if (D.hq % D.hkv != 0) return SAGE_ERR_GQA;
    const int64_t* st[4] = {D.q_stride, D.k_stride, D.v_stride, D.o_stride};
    for (auto s : st)
        for (int i = 0; i < 3; ++i)
            if (s[i] < 0 || s[i] % 8 != 0) return SAGE_ERR_STRIDE;

    Plan p;
    p.varlen = varlen;
    p.d = D.head_dim;
    p.hq = D.hq;
    p.hkv = D.hkv;
    p.group = D.hq / D.hkv;
    p.causal = D.is_causal;
    p.smooth_q = D.smooth_q != 0;
    p.smooth_q_blk = D.smooth_q == SAGE_SMOOTH_Q_BLOCK;
    p.smooth_k = D.smooth_k;
    p.smooth_v = D.smooth_v;
    p.pv_half = D.pv_mode == SAGE_PV_HALF;
    p.kv_split_req = D.kv_split;
    p.qb = D.qk_block == 32 ? 32 : QBLK;
    p.sm_scale = D.sm_scale > 0.0f ? D.sm_scale : 1.0f / std::sqrt((float)D.head_dim);
    if (varlen) {
        if (cuq[0] != 0 || cuk[0] != 0) return SAGE_ERR_SEQLENS;
        p.S = nseq;
        for (int s = 0; s < nseq; ++s) {
            const int64_t lq = (int64_t)cuq[s + 1] - cuq[s];
            const int64_t lk = (int64_t)cuk[s + 1] - cuk[s];
            if (lq < 0 || lk < 0 || lq > (1 << 24) || lk > (1 << 24)) return SAGE_ERR_SEQLENS;
            p.nq.push_back((int32_t)lq);
            p.nkv.push_back((int32_t)lk);
            p.tq.push_back(cuq[s]);
            p.tk.push_back(cuk[s]);
        }
        p.total_q = nseq > 0 ? cuq[nseq] : 0;
    } else {
        p.S = D.batch;
        p.nq.assign(p.S, D.nq);
        p.nkv.assign(p.S, D.nkv);
        p.tq.assign(p.S, 0);
        p.tk.assign(p.S, 0);
        p.total_q = (int64_t)D.batch * D.nq;
    }
    for (int s = 0; s < p.S; ++s) {
        p.rq.push_back(p.rows_q);
        p.rk.push_back(p.rows_k);
        p.rows_q += round_up(p.nq[s], QBLK);
        p.rows_k += round_up(p.nkv[s], KVT);
        p.max_nkv = std::max(p.max_nkv, p.nkv[s]);
    }
    p.rows_total = varlen ? (int64_t)p.hq * p.total_q : (int64_t)p.S * p.hq * D.nq;
    // strides: all-zero triple = contiguous in the layout
    const int64_t d = D.head_dim;
    auto fill = [&](const int64_t* in, int heads, int64_t n, Strides* o) {
        if (in[0] || in[1] || in[2]) {
            *o = Strides{in[0], in[1], in[2]};
            return;
        }
        if (D.layout == SAGE_HND) {
            // dense [B,H,N,d]; varlen [H,T,d]
            *o = Strides{heads * n * d, n * d, d};
        } else {
            // dense [B,N,H,d]; varlen [T,H,d]
            *o = Strides{n * heads * d, d, heads * d};
        }
    };
    int64_t tot_k = 0;
    if (varlen) tot_k = nseq > 0 ? cuk[nseq] : 0;
    fill(D.q_stride, D.hq, varlen ? p.total_q : D.nq, &p.qs);
    fill(D.k_stride, D.hkv, varlen ? tot_k : D.nkv, &p.ks);
    fill(D.v_stride, D.hkv, varlen ? tot_k : D.nkv, &p.vs);
    fill(D.o_stride, D.hq, varlen ? p.total_q : D.nq, &p.os);
    resolve_split(&p);
    *out = std::move(p);
    return SAGE_OK;
}

// gfx950 check, cached per device.
sage_status check_arch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
    static std::mutex mu;
    static std::vector<int> known;   // 0 unknown, 1 ok, 2 bad
    std::lock_guard<std::mutex> lock(mu);
    if ((int)known.size() <= dev) known.resize(dev + 1, 0);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SAGE_ERR_HIP;
        known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return known[dev] == 1 ? SAGE_OK : SAGE_ERR_ARCH;
}

// Kernel parameter blocks: one per group of at most MAXSEQ sequences.  Dense
// problems need a single uniform table.  Varlen sequences are ordered by
// descending work so that the heaviest are dispatched first.
std::vector<KParams> make_params(const Plan& p) {
    KParams base{};
    base.d = p.d;
    base.hq = p.hq;
    base.hkv = p.hkv;
    base.group = p.group;
    base.causal = p.causal;
    base.pv_half = p.pv_half;
    base.qb = p.qb;
    base.sm_scale = p.sm_scale;
    base.sml2 = (float)((double)p.sm_scale * 1.4426950408889634);
    base.qs = p.qs;
    base.ks = p.ks;
    base.vs = p.vs;
    base.os = p.os;
    base.kv_tiles = p.kv_split / KVT;
    base.nsplit = p.kv_split ? p.nsplit : 1;
    base.rows_total = p.rows_total;
    base.bqs = p.smooth_q_blk;
    std::vector<KParams> out;
    if (!p.varlen) {
        if (p.S == 0) return out;
        KParams k = base;
        k.lse_hstride = p.nq[0];
        k.tab.n = p.S;
        k.tab.uniform = 1;
        k.tab.nq[0] = p.nq[0];
        k.tab.nkv[0] = p.nkv[0];
        out.push_back(k);
        return out;
    }
    std::vector<int> order(p.S);
    for (int s = 0; s < p.S; ++s) order[s] = s;
    auto cost = [&](int s) {
        const double nq = p.nq[s], nkv = p.nkv[s];
        return p.causal ? nq * nkv - 0.5 * std::min(nq, nkv) * std::min(nq, nkv) : nq * nkv;
    };
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cost(a) > cost(b); });
    for (size_t i0 = 0; i0 < order.size(); i0 += MAXSEQ) {
        KParams k = base;
        k.lse_hstride = p.total_q;
        k.tab.uniform = 0;
        k.tab.n = (int)std::min<size_t>(MAXSEQ, order.size() - i0);
        for (int j = 0; j < k.tab.n; ++j) {
            const int s = order[i0 + j];
            k.tab.nq[j] = p.nq[s];
            k.tab.nkv[j] = p.nkv[s];
            k.tab.tq[j] = p.tq[s];
            k.tab.tk[j] = p.tk[s];
            k.tab.rq[j] = p.rq[s];
            k.tab.rk[j] = p.rk[s];
            k.tab.sid[j] = s;
            k.tab.lse_base[j] = p.tq[s];
        }
        out.push_back(k);
    }
    return out;
}

// The split of the key range.  An explicit kv_split is used as given (no
// split when it covers the longest key range).  SAGE_KV_SPLIT_AUTO:
// * decode shapes (GQA group x queries of every sequence within one wave's
//   DEC_ROWS rows) run one wave per (sequence, kv head, split); the rule aims
//   at one round of the grid, 256 compute units x decode_waves_per_cu waves
//   (4 for FP8 V, 3 for 16-bit V at d = 128), and at least two splits, with
//   at least 4 key tiles (512 keys) per split;
// * other shapes split only when the unsplit grid has fewer workgroups than
//   MI355X has compute units (256); it then aims at 512 workgroups, with at
//   least 4 key tiles per split.
// The rule depends on the problem only, never on the device it runs on.
void resolve_split(Plan* p) {
    int32_t ks = 0;
    const int32_t tiles_max = (p->max_nkv + KVT - 1) / KVT;
    int32_t max_nq = 0;
    for (int s = 0; s < p->S; ++s) max_nq = std::max(max_nq, p->nq[s]);
    if (p->kv_split_req > 0) {
        ks = p->kv_split_req;
    } else if (p->kv_split_req == SAGE_KV_SPLIT_AUTO && tiles_max > 0) {
        int64_t want = 0;
        if ((int64_t)p->group * std::max(max_nq, 1) <= DEC_ROWS) {
            const int64_t units = (int64_t)p->S * p->hkv;
            const int64_t round =
                (int64_t)NUM_CU * decode_waves_per_cu(p->d, p->pv_half, p->smooth_q, p->group);
            want = std::max<int64_t>(2, round / units);
        } else {
            Plan tmp = *p;
            tmp.kv_split = 0;
            int64_t base = 0;
            for (const KParams& P : make_params(tmp)) base += attn_base_wgs(P);
            if (base > 0 && base < 256) want = (512 + base - 1) / base;
        }
        if (want > 0) {
            const int32_t tps = std::max<int32_t>(4, (int32_t)((tiles_max + want - 1) / want));
            ks = tps * KVT;
        }
    }
    if (ks >= p->max_nkv) ks = 0;   // one split: the plain kernel
    p->kv_split = ks;
    p->nsplit = ks ? (p->max_nkv + ks - 1) / ks : 1;
}

// Blocks of a launch over (head, 64-token chunk) pairs for one table.
int chunk_blocks(const KParams& k, bool is_q, int heads, bool padded) {
    int tot = 0;
    const int n = k.tab.uniform ? 1 : k.tab.n;
    for (int s = 0; s < n; ++s) {
        const int len = is_q ? k.tab.nq[s] : k.tab.nkv[s];
        const int np = padded ? round_up(len, is_q ? QBLK : KVT) : round_up(len, QBLK);
        tot += heads * (np / QBLK);
    }
    return k.tab.uniform ? tot * k.tab.n : tot;
}

int tab_seqs(const KParams& k) { return k.tab.n; }

// Workgroups of a statistics job over Q (is_q) or K/V.
int stat_blocks(const KParams& k, bool is_q, int heads) {
    const int cpw = stat_chunks_per_wg(k.d);
    int tot = 0;
    const int n = k.tab.uniform ? 1 : k.tab.n;
    for (int s = 0; s < n; ++s) {
        const int len = is_q ? k.tab.nq[s] : k.tab.nkv[s];
        const int nch = (len + QBLK - 1) / QBLK;
        tot += heads * ((nch + cpw - 1) / cpw);
    }
    return k.tab.uniform ? tot * k.tab.n : tot;
}

#define SAGE_TRY(x)                                  \
    do {                                             \
        if ((x) != hipSuccess) return SAGE_ERR_HIP;  \
    } while (0)

// The pre-pass.  `bufs` are the destination tensors, `sc` the scratch area.
// With skip_q the Q codes are left to the fused kernel (its means are still
// formed here).
sage_status run_prepass(const Plan& p, const std::vector<KParams>& kp, int dtype, const void* q,
                        const void* k, const void* v, const sage_quant_bufs& b, uint8_t* sc,
                        const WsLayout& w, hipStream_t st, bool skip_q = false) {
    float* part_q = reinterpret_cast<float*>(sc + w.part_q);
    float* part_k = reinterpret_cast<float*>(sc + w.part_k);
    float* part_v = reinterpret_cast<float*>(sc + w.part_v);
    float* part_vmax = reinterpret_cast<float*>(sc + w.part_vmax);
    float* v_amax = reinterpret_cast<float*>(sc + w.v_amax);
    for (const KParams& P : kp) {
        const int kblocks = stat_blocks(P, false, p.hkv);
        const int qblocks = stat_blocks(P, true, p.hq);
        const int nseq = tab_seqs(P);
        // finalize workgroups: one per sequence, head and FIN_CH channels
        const int fin_wgs = nseq * p.hkv * (p.d / FIN_CH);
        const int fin_wgs_q = nseq * p.hq * (p.d / FIN_CH);
        // 1. chunk statistics: the means that are needed, and the absolute
        //    maxima of V when V is not smoothed (else they need mu_v first)
        StatJobs sj{};
        FinJobs fj{};
        int n = 0;
        if (p.smooth_k) {
            sj.j[n] = StatJob{static_cast<const uint16_t*>(k), P.ks, nullptr, part_k, 1, p.hkv,
                              STAT_SUM, kblocks};
            fj.j[n++] = FinJob{part_k, b.mu_k, nullptr, nullptr, 0, p.hkv, STAT_SUM, fin_wgs};
        }
        if (p.smooth_q) {
            sj.j[n] = StatJob{static_cast<const uint16_t*>(q), P.qs, nullptr, part_q, 0, p.hq,
                              STAT_SUM, qblocks};
            fj.j[n++] = FinJob{part_q, b.mu_q, nullptr, nullptr, 1, p.hq, STAT_SUM, fin_wgs_q};
        }
        if (p.smooth_v) {
            sj.j[n] = StatJob{static_cast<const uint16_t*>(v), P.vs, nullptr, part_v, 2, p.hkv,
                              STAT_SUM, kblocks};
            fj.j[n++] = FinJob{part_v, b.mu_v, nullptr, nullptr, 0, p.hkv, STAT_SUM, fin_wgs};
        } else if (!p.pv_half) {
            sj.j[n] = StatJob{static_cast<const uint16_t*>(v), P.vs, nullptr, part_vmax, 2, p.hkv,
                              STAT_ABSMAX, kblocks};
            fj.j[n++] = FinJob{part_vmax, nullptr, v_amax, b.v_scale, 0, p.hkv, STAT_ABSMAX,
                               fin_wgs};
        }
        SAGE_TRY(launch_stats(P, dtype, sj, st));
        SAGE_TRY(launch_finalize(P, fj, st));
        if (p.smooth_v && !p.pv_half) {
            // 2. absolute maxima of V - mu_v
            StatJobs sv{};
            sv.j[0] = StatJob{static_cast<const uint16_t*>(v), P.vs, b.mu_v, part_vmax, 2, p.hkv,
                              STAT_ABSMAX, kblocks};
            FinJobs fv{};
            fv.j[0] = FinJob{part_vmax, nullptr, v_amax, b.v_scale, 0, p.hkv, STAT_ABSMAX,
                             fin_wgs};
            SAGE_TRY(launch_stats(P, dtype, sv, st));
            SAGE_TRY(launch_finalize(P, fv, st));
        }
        // 3. every code and scale in one launch
        QuantArgs qa{};
        qa.q = static_cast<const uint16_t*>(q);
        qa.k = static_cast<const uint16_t*>(k);
        qa.v = static_cast<const uint16_t*>(v);
        qa.mu_q = p.smooth_q ? b.mu_q : nullptr;
        qa.mu_k = p.smooth_k ? b.mu_k : nullptr;
        qa.mu_v = p.smooth_v ? b.mu_v : nullptr;
        qa.v_amax = v_amax;
        qa.q_codes = b.q_codes;
        qa.k_codes = b.k_codes;
        qa.v_codes = b.v_codes;
        qa.q_scale = b.q_scale;
        qa.k_scale = b.k_scale;
        qa.delta_s = p.smooth_q ? b.delta_s : nullptr;
        qa.mu_qb = p.smooth_q_blk ? b.mu_qb : nullptr;
        qa.mq_code = p.smooth_q_blk ? b.mu_q_code : nullptr;
        qa.mq_scale = p.smooth_q_blk ? b.mu_q_cscale : nullptr;
        qa.nq = skip_q ? 0 : chunk_blocks(P, true, p.hq, true);
        qa.nk = chunk_blocks(P, false, p.hkv, true);
        // 16-bit V: 64-token chunks (128-byte rows already); E4M3 V: one
        // 128-token key tile per workgroup
        qa.nv = chunk_blocks(P, false, p.hkv, true) / (p.pv_half ? 1 : KVT / QBLK);
        qa.v_half = p.pv_half;
        SAGE_TRY(launch_quant(P, dtype, qa, st));
    }
    return SAGE_OK;
}

uint8_t* align_up(void* p) {
    uintptr_t u = reinterpret_cast<uintptr_t>(p);
    return reinterpret_cast<uint8_t*>((u + ALIGN - 1) / ALIGN * ALIGN);
}

sage_quant_bufs bufs_in_ws(const Plan& p, uint8_t* ws, const WsLayout& w) {
    sage_quant_bufs b{};
    b.mu_q = p.smooth_q ? reinterpret_cast<float*>(ws + w.mu_q) : nullptr;
    b.mu_k = p.smooth_k ? reinterpret_cast<float*>(ws + w.mu_k) : nullptr;
    b.mu_v = p.smooth_v ? reinterpret_cast<float*>(ws + w.mu_v) : nullptr;
    b.q_codes = reinterpret_cast<int8_t*>(ws + w.q_codes);
    b.q_scale = reinterpret_cast<float*>(ws + w.q_scale);
    b.k_codes = reinterpret_cast<int8_t*>(ws + w.k_codes);
    b.k_scale = reinterpret_cast<float*>(ws + w.k_scale);
    b.v_codes = reinterpret_cast<uint8_t*>(ws + w.v_codes);
    b.v_scale = p.pv_half ? nullptr : reinterpret_cast<float*>(ws + w.v_scale);
    b.delta_s = p.smooth_q ? reinterpret_cast<float*>(ws + w.delta_s) : nullptr;
    b.mu_qb = p.smooth_q_blk ? reinterpret_cast<float*>(ws + w.mu_qb) : nullptr;
    b.mu_q_code = p.smooth_q_blk ? reinterpret_cast<int8_t*>(ws + w.mu_q_code) : nullptr;
    b.mu_q_cscale = p.smooth_q_blk ? reinterpret_cast<float*>(ws + w.mu_q_cscale) : nullptr;
    return b;
}

// The fused kernel over every parameter block, then (split key range) the
// merge of the partials.  q_raw: the kernel quantizes this Q itself (null:
// it reads the codes in `b`).
sage_status run_attn(const Plan& p, std::vector<KParams> kp, int dtype, const sage_quant_bufs& b,
                     const float* ds, const float* mu_v, void* o, float* lse, float* part_o,
                     float* part_ml, hipStream_t st, const void* q_raw = nullptr) {
    for (KParams& P : kp) {
        P.part_o = part_o;
        P.part_ml = part_ml;
        P.q_raw = static_cast<const uint16_t*>(q_raw);
        SAGE_TRY(launch_attn(P, dtype, b.q_codes, b.q_scale, b.k_codes, b.k_scale, b.v_codes,
                             b.v_scale, ds, mu_v, o, lse, p.smooth_q_blk ? b.mu_q_code : nullptr,
                             p.smooth_q_blk ? b.mu_q_cscale : nullptr, st));
    }
    if (p.kv_split && p.rows_total > 0) {
        MergeArgs m{};
        m.part_o = part_o;
        m.part_ml = part_ml;
        m.rows_total = p.rows_total;
        m.nsplit = p.nsplit;
        m.d = p.d;
        m.hq = p.hq;
        m.nq = p.varlen ? 0 : p.nq[0];
        m.varlen = p.varlen;
        m.total_q = p.total_q;
        m.poff = p.pv_half ? 0.0f : (float)std::log2(448.0);
        m.os = p.os;
        m.o = o;
        m.lse = lse;
        SAGE_TRY(launch_merge(m, dtype, st));
    }
    return SAGE_OK;
}

sage_status forward(const sage_attn_desc* desc, const int32_t* cuq, const int32_t* cuk,
                    int32_t nseq, bool varlen, const void* q, const void* k, const void* v,
                    void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    sage_status e = make_plan(desc, cuq, cuk, nseq, varlen, &p);
    if (e != SAGE_OK) return e;
    const bool empty = p.S == 0 || p.total_q == 0;
    if (!empty && (!q || !o || (p.rows_k > 0 && (!k || !v)) || !ws)) return SAGE_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return SAGE_ERR_ALIGN;
    const WsLayout w = ws_layout(p, true);
    if (!empty && ws_bytes < w.total) return SAGE_ERR_WORKSPACE;
    if ((e = check_arch()) != SAGE_OK) return e;
    if (empty) return SAGE_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* base = align_up(ws);
    const sage_quant_bufs b = bufs_in_ws(p, base, w);
    const std::vector<KParams> kp = make_params(p);
    // The fused kernel quantizes Q itself (Q is read once, by the kernel that
    // needs it), unless Q is smoothed (with the score bias that measured
    // slower than the pre-pass work it saves) or a launch runs the decode
    // kernel, which reads codes.
    bool fuse_q = !p.smooth_q;
    for (const KParams& P : kp) fuse_q = fuse_q && !use_decode_kernel(P);
    if ((e = run_prepass(p, kp, desc->dtype, q, k, v, b, base, w, st, fuse_q)) != SAGE_OK)
        return e;
    return run_attn(p, kp, desc->dtype, b, p.smooth_q ? b.delta_s : nullptr,
                    p.smooth_v ? b.mu_v : nullptr, o, lse,
                    reinterpret_cast<float*>(base + w.split_o),
                    reinterpret_cast<float*>(base + w.split_ml), st, fuse_q ? q : nullptr);
}

}  // namespace

extern "C" {

void sage_desc_init(sage_attn_desc* desc, int32_t dtype, int32_t layout, int32_t batch,
                    int32_t hq, int32_t hkv, int32_t nq, int32_t nkv, int32_t head_dim) {
    if (!desc) return;
    std::memset(desc, 0, sizeof(*desc));
    desc->dtype = dtype;
    desc->layout = layout;
    desc->batch = batch;
    desc->hq = hq;
    desc->hkv = hkv;
    desc->nq = nq;
    desc->nkv = nkv;
    desc->head_dim = head_dim;
    desc->smooth_k = 1;
    desc->sm_scale = 0.0f;
}

sage_status sage_quant_buf_sizes(const sage_attn_desc* desc, const int32_t* cuq,
                                 const int32_t* cuk, int32_t nseq, sage_quant_sizes* sizes) {
    if (!sizes) return SAGE_ERR_NULL;
    Plan p;
    const sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    *sizes = quant_sizes(p);
    return SAGE_OK;
}

sage_status sage_workspace_size(const sage_attn_desc* desc, const int32_t* cuq,
                                const int32_t* cuk, int32_t nseq, size_t* bytes) {
    if (!bytes) return SAGE_ERR_NULL;
    Plan p;
    const sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    *bytes = ws_layout(p, true).total;
    return SAGE_OK;
}

sage_status sage_quant_qkv(const sage_attn_desc* desc, const void* q, const void* k,
                           const void* v, const int32_t* cuq, const int32_t* cuk, int32_t nseq,
                           const sage_quant_bufs* out, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    if (!out) return SAGE_ERR_NULL;
    const bool empty = p.S == 0;
    if (!empty) {
        if (!q || !k || !v || !ws || !out->q_codes || !out->q_scale || !out->k_codes ||
            !out->k_scale || !out->v_codes || (!p.pv_half && !out->v_scale) ||
            (p.smooth_q && !out->mu_q) ||
            (p.smooth_k && !out->mu_k) || (p.smooth_v && !out->mu_v) ||
            (p.smooth_q && !out->delta_s) ||
            (p.smooth_q_blk && (!out->mu_qb || !out->mu_q_code || !out->mu_q_cscale)))
            return SAGE_ERR_NULL;
    }
    const void* ptrs[] = {q, k, v, out->q_codes, out->k_codes, out->v_codes, out->q_scale,
                          out->k_scale, out->v_scale, out->mu_q, out->mu_k, out->mu_v,
                          out->delta_s, out->mu_qb, out->mu_q_code, out->mu_q_cscale};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return SAGE_ERR_ALIGN;
    const WsLayout w = ws_layout(p, false);
    if (!empty && ws_bytes < w.total) return SAGE_ERR_WORKSPACE;
    if ((e = check_arch()) != SAGE_OK) return e;
    if (empty) return SAGE_OK;
    const std::vector<KParams> kp = make_params(p);
    return run_prepass(p, kp, desc->dtype, q, k, v, *out, align_up(ws), w,
                       static_cast<hipStream_t>(stream));
}

sage_status sage_attn_fwd(const sage_attn_desc* desc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                          void* stream) {
    return forward(desc, nullptr, nullptr, 0, false, q, k, v, o, lse, ws, ws_bytes, stream);
}

sage_status sage_attn_fwd_noalloc(const sage_attn_desc* desc, const void* q, const void* k,
                                  const void* v, void* o, float* lse, void* stream) {
    // the checks of sage_attn_fwd, then the workspace: the static array of
    // this device (no allocation of any kind)
    Plan p;
    sage_status e = make_plan(desc, nullptr, nullptr, 0, false, &p);
    if (e != SAGE_OK) return e;
    if (ws_layout(p, true).total > NOALLOC_WS_MAX) return SAGE_ERR_WORKSPACE;
    if ((e = check_arch()) != SAGE_OK) return e;
    void* ws = nullptr;
    SAGE_TRY(noalloc_workspace(&ws));
    return forward(desc, nullptr, nullptr, 0, false, q, k, v, o, lse, ws, NOALLOC_WS_MAX, stream);
}

sage_status sage_attn_fwd_varlen(const sage_attn_desc* desc, const int32_t* cuq,
                                 const int32_t* cuk, int32_t nseq, const void* q, const void* k,
                                 const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                                 void* stream) {
    return forward(desc, cuq, cuk, nseq, true, q, k, v, o, lse, ws, ws_bytes, stream);
}

sage_status sage_attn_fwd_quantized(const sage_attn_desc* desc, const int32_t* cuq,
                                    const int32_t* cuk, int32_t nseq, const sage_quant_bufs* b,
                                    void* o, float* lse, void* ws, size_t ws_bytes,
                                    void* stream) {
    Plan p;
    sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    if (!b) return SAGE_ERR_NULL;
    const bool empty = p.S == 0 || p.total_q == 0;
    if (!empty && (!o || !b->q_codes || !b->q_scale || !b->k_codes || !b->k_scale ||
                   !b->v_codes || (!p.pv_half && !b->v_scale) || (p.smooth_q && !b->delta_s) ||
                   (p.smooth_v && !b->mu_v) ||
                   (p.smooth_q_blk && (!b->mu_q_code || !b->mu_q_cscale))))
        return SAGE_ERR_NULL;
    const void* ptrs[] = {o, b->q_codes, b->k_codes, b->v_codes, b->q_scale, b->k_scale,
                          b->v_scale, b->mu_v, b->delta_s, b->mu_q_code, b->mu_q_cscale};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return SAGE_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return SAGE_ERR_ALIGN;
    const WsLayout w = ws_layout_fused(p);
    if (!empty && w.total > 0 && !ws) return SAGE_ERR_NULL;
    if (!empty && ws_bytes < w.total) return SAGE_ERR_WORKSPACE;
    if ((e = check_arch()) != SAGE_OK) return e;
    if (empty) return SAGE_OK;
    uint8_t* base = w.total ? align_up(ws) : nullptr;
    return run_attn(p, make_params(p), desc->dtype, *b, p.smooth_q ? b->delta_s : nullptr,
                    p.smooth_v ? b->mu_v : nullptr, o, lse,
                    base ? reinterpret_cast<float*>(base + w.split_o) : nullptr,
                    base ? reinterpret_cast<float*>(base + w.split_ml) : nullptr,
                    static_cast<hipStream_t>(stream));
}

sage_status sage_kv_split_size(const sage_attn_desc* desc, const int32_t* cuq,
                               const int32_t* cuk, int32_t nseq, int32_t* keys_per_split) {
    if (!keys_per_split) return SAGE_ERR_NULL;
    Plan p;
    const sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    *keys_per_split = p.kv_split;
    return SAGE_OK;
}

sage_status sage_debug_qk_int32(const sage_attn_desc* desc, const int32_t* cuq,
                                const int32_t* cuk, int32_t nseq, const sage_quant_bufs* bufs,
                                int32_t* s_out, void* stream) {
    Plan p;
    sage_status e = make_plan(desc, cuq, cuk, nseq, cuq != nullptr, &p);
    if (e != SAGE_OK) return e;
    if (!bufs) return SAGE_ERR_NULL;
    if (p.S > 0 && (!bufs->q_codes || !bufs->k_codes || !s_out)) return SAGE_ERR_NULL;
    if (!aligned16(bufs->q_codes) || !aligned16(bufs->k_codes) || !aligned16(s_out))
        return SAGE_ERR_ALIGN;
    if ((e = check_arch()) != SAGE_OK) return e;
    std::vector<int64_t> gbase(p.S + 1, 0);
    for (int s = 0; s < p.S; ++s) gbase[s + 1] = gbase[s] + (int64_t)p.hq * p.nq[s] * p.nkv[s];
    for (KParams P : make_params(p)) {
        P.kv_tiles = 0;           // the dump covers every key of every row
        P.nsplit = 1;
        P.causal = 0;
        if (!P.tab.uniform)
            for (int j = 0; j < P.tab.n; ++j) P.tab.dump0[j] = gbase[P.tab.sid[j]];
        SAGE_TRY(launch_qk_dump(P, bufs->q_codes, bufs->k_codes, s_out,
                                static_cast<hipStream_t>(stream)));
    }
    return SAGE_OK;
}

sage_status sage_debug_e4m3_encode(uint32_t first, uint32_t count, uint8_t* out, void* stream) {
    if (count > 0 && !out) return SAGE_ERR_NULL;
    if (!aligned16(out)) return SAGE_ERR_ALIGN;
    if ((uint64_t)first + count > (uint64_t{1} << 32)) return SAGE_ERR_SHAPE;
    sage_status e = check_arch();
    if (e != SAGE_OK) return e;
    SAGE_TRY(launch_e4m3_dump(first, count, out, static_cast<hipStream_t>(stream)));
    return SAGE_OK;
}

sage_status sage_micro_rate(int32_t op, int32_t reps, double* rate, void* stream) {
    if (!rate) return SAGE_ERR_NULL;
    if (op < SAGE_MICRO_I8 || op > SAGE_MICRO_FMA) return SAGE_ERR_FLAGS;
    if (reps < 1 || reps > (1 << 20)) return SAGE_ERR_SHAPE;
    sage_status e = check_arch();
    if (e != SAGE_OK) return e;
    SAGE_TRY(micro_rate(op, reps, rate, static_cast<hipStream_t>(stream)));
    return SAGE_OK;
}

const char* sage_status_string(int32_t s) {
    switch (s) {
        case SAGE_OK: return "ok";
        case SAGE_ERR_NULL: return "null pointer";
        case SAGE_ERR_DTYPE: return "unsupported dtype";
        case SAGE_ERR_LAYOUT: return "unsupported layout";
        case SAGE_ERR_HEAD_DIM: return "head_dim must be 64, 96 or 128";
        case SAGE_ERR_SHAPE: return "invalid shape";
        case SAGE_ERR_GQA: return "hq must be a multiple of hkv";
        case SAGE_ERR_STRIDE: return "invalid stride";
        case SAGE_ERR_ALIGN: return "pointer not 16-byte aligned";
        case SAGE_ERR_WORKSPACE: return "workspace too small";
        case SAGE_ERR_SEQLENS: return "invalid cu_seqlens";
        case SAGE_ERR_ARCH: return "device is not gfx950";
        case SAGE_ERR_HIP: return "HIP runtime error";
        case SAGE_ERR_FLAGS: return "invalid flag, pv_mode, kv_split or qk_block";
    }
    return "unknown status";
}

int32_t sage_abi_version(void) { return SAGE_ABI_VERSION; }

}  // extern "C"
