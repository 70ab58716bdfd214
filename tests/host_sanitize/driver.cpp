// Seeded fuzzing of the library's host layer (argument validation, size and
// extent arithmetic, the varlen plan builder, the THD planner and its first-
// position table), built with AddressSanitizer and UndefinedBehaviorSanitizer
// for the host only.  Device pointers are fake addresses: nothing is launched
// (the stubs count the launches the validation lets through).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "cam.h"

namespace cam {
extern long g_launches;
}

static std::mt19937_64 rng(20260913);

static int64_t pick(std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); }

static int64_t any_size()
{
    return pick({0, 1, 2, 3, 7, 8, 16, 63, 64, 65, 128, 512, 1000, 4096, 65535, 65536, 131072, (1LL << 31) - 1,
                 1LL << 31, (1LL << 32) + 1, 1LL << 40, (1LL << 62) + 3, INT64_MAX, -1, -2, INT64_MIN});
}

static const void* any_ptr()
{
    const uintptr_t base = uintptr_t(0x7F0000000000ull) + (rng() % 64) * (uintptr_t(1) << 34);
    return reinterpret_cast<const void*>(base + pick({0, 0, 0, 2, 4, 8, 16}));
}

static void fuzz_abi(int rounds)
{
    for (int i = 0; i < rounds; ++i) {
        const cam_dtype dt = cam_dtype(pick({0, 1, 2, 7}));
        const int sd = int(pick({0, 1, 2}));
        void* p = const_cast<void*>(any_ptr());
        void* q = const_cast<void*>(any_ptr());
        const int32_t* ci = static_cast<const int32_t*>(any_ptr());
        const int64_t* cl = static_cast<const int64_t*>(any_ptr());
        float* f = static_cast<float*>(const_cast<void*>(any_ptr()));
        int64_t a[24];
        for (int64_t& v : a)
            v = any_size();
        switch (i % 17) {
        case 0: ulysses_seq_to_head(p, q, a[0], a[1], a[2], a[3], a[4], dt, nullptr); break;
        case 1: ulysses_head_to_seq(p, q, a[0], a[1], a[2], a[3], a[4], dt, nullptr); break;
        case 2: ulysses_seq_to_head_varlen(p, q, ci, ci, cl, a[0], a[1], a[2], a[3], a[4], a[5], dt, nullptr); break;
        case 3: ulysses_head_to_seq_varlen(p, q, ci, ci, cl, a[0], a[1], a[2], a[3], a[4], a[5], dt, nullptr); break;
        case 4: ulysses_seq_to_head_spans(p, q, ci, ci, ci, cl, a[0], a[1], a[2], a[3], a[4], a[5], dt, nullptr); break;
        case 5: lse_pack_bytes(a[0], a[1], a[2], a[3], sd, dt); break;
        case 6:
            lse_pack(p, a[0], a[1], a[2], f, a[3], a[4], a[5], f, a[6], a[7], a[8], a[9], a[10], a[11], a[12], sd, dt, q,
                     nullptr);
            break;
        case 7: lse_combine_packed(p, a[0], a[1], a[2], a[3], sd, dt, q, f, nullptr); break;
        case 8:
            lse_combine(p, a[0], a[1], a[2], f, a[3], a[4], a[5], a[6], a[7], a[8], a[9], dt, q, a[10], a[11], f, a[12],
                        a[13], nullptr);
            break;
        case 9:
            lse_combine_varlen(p, a[0], a[1], a[2], f, a[3], a[4], a[5], a[6], a[7], a[8], a[9], dt, q, a[10], a[11], f,
                               a[12], a[13], ci, a[14], nullptr);
            break;
        case 10:
            lse_combine_planned(p, a[0], a[1], a[2], f, a[3], a[4], a[5], a[6], a[7], a[8], a[9], dt, q, a[10], a[11],
                                f, a[12], a[13], ci, ci, a[14], nullptr);
            break;
        case 11: lse_combine_packed_seq(p, a[0], a[1], a[2], a[3], sd, dt, q, f, nullptr); break;
        case 12:
            lse_combine_varlen_seq(p, a[0], a[1], a[2], f, a[3], a[4], a[5], a[6], a[7], a[8], a[9], dt, q, f, ci, ci,
                                   cl, a[10], nullptr);
            break;
        case 13:
            lse_merge(f, a[0], a[1], f, a[2], a[3], p, a[4], a[5], f, a[6], a[7], a[8], a[9], a[10], dt, q, a[11], a[12],
                      nullptr);
            break;
        case 14:
            lse_combine_backward(p, a[0], a[1], a[2], f, a[3], a[4], a[5], a[6], a[7], a[8], a[9], dt, q, a[10], a[11],
                                 f, a[12], a[13], p, a[14], a[15], a[16], f, a[17], a[18], a[19], nullptr);
            break;
        case 15: qkv_projection_head_sharded(p, q, p, a[0], a[1], a[2], a[3], a[4], a[5], dt, nullptr); break;
        case 16:
            cam_ablation_seq_to_head_lds(p, q, a[0], a[1], a[2], a[3], a[4], dt, a[5], nullptr);
            cam_copy(p, q, a[6], nullptr);
            break;
        }
    }
}

// random packed batches: lengths in blocks, some zero-length
static std::vector<int32_t> batch(int64_t b, int64_t nseq, int64_t max_blocks)
{
    std::vector<int32_t> cu(size_t(nseq) + 1, 0);
    for (int64_t i = 0; i < nseq; ++i)
        cu[size_t(i) + 1] = cu[size_t(i)] + int32_t(b * int64_t(rng() % uint64_t(max_blocks + 1)));
    return cu;
}

static void fuzz_plans(int rounds)
{
    long ok = 0;
    for (int i = 0; i < rounds; ++i) {
        const int64_t nseq = 1 + int64_t(rng() % 24);
        const int64_t P = 1 + int64_t(rng() % 9);
        const int64_t b = pick({1, 2, 4, 64});
        std::vector<int32_t> cu = batch(b, nseq, 40);
        // the per-sequence split's plan
        std::vector<int32_t> rank_cu(size_t(P * (nseq + 1)));
        std::vector<int64_t> rank_off(size_t(P + 1));
        ulysses_varlen_plan(cu.data(), nseq, P, rank_cu.data(), rank_off.data());
        // the THD planner, every configuration field varied
        cam_thd_planner_config cfg;
        cfg.block_size = b;
        cfg.min_split_tokens = b * pick({1, 2, 8, 64});
        cfg.max_chunks_per_rank = pick({1, 4, 64});
        cfg.token_weight = double(pick({0, 1, 3}));
        cfg.causal_weight = double(pick({0, 1}));
        cfg.mode = pick({0, 1});
        int64_t max_spans = cfg.max_chunks_per_rank * P + nseq + 2;
        if (i % 4 == 3) {  // malformed requests: each must be refused without a write out of bounds
            switch (rng() % 7) {
            case 0: cfg.block_size = pick({0, -1, 3, INT64_MAX}); break;
            case 1: cfg.min_split_tokens = pick({0, -64, b + 1, INT64_MAX}); break;
            case 2: cfg.max_chunks_per_rank = pick({0, -1, INT64_MAX}); break;
            case 3: cfg.token_weight = pick({0, 1}) ? -1.0 : 1e308 * 10; cfg.causal_weight = -0.5; break;
            case 4: max_spans = int64_t(rng() % uint64_t(max_spans)); break;   // a span table too small
            case 5: if (nseq > 1) cu[1] = cu[2] + 1; break;                       // decreasing cu_seqlens
            case 6: cu[size_t(nseq)] += int32_t(b / 2 + (b == 1)); break;        // a length off the blocks
            }
        }
        const size_t ns = static_cast<size_t>(max_spans > 0 ? max_spans : 0);
        std::vector<int32_t> span_start(ns + 1), span_rank(ns), span_local(ns);
        std::vector<int64_t> roff(static_cast<size_t>(P) + 1);
        std::vector<double> cost(static_cast<size_t>(P) + 0);
        int64_t n_spans = 0;
        int32_t chosen = 0;
        const cam_status st = thd_plan(cu.data(), nseq, P, &cfg, max_spans, span_start.data(), span_rank.data(),
                                       span_local.data(), roff.data(), cost.data(), &n_spans, &chosen);
        if (st == CAM_OK) {
            ++ok;
            std::vector<int32_t> first(size_t(P * nseq));
            thd_plan_first_positions(cu.data(), nseq, P, span_start.data(), span_rank.data(), n_spans, first.data());
        }
    }
    std::printf("plans: %d batches, %ld planned\n", rounds, ok);
}

int main(int argc, char** argv)
{
    // optional: seed, ABI calls, planner batches
    if (argc > 1)
        rng.seed(std::strtoull(argv[1], nullptr, 10));
    const int calls = argc > 2 ? std::atoi(argv[2]) : 200000;
    const int plans = argc > 3 ? std::atoi(argv[3]) : 3000;
    fuzz_abi(calls);
    fuzz_plans(plans);
    std::printf("launch records accepted: %ld\n", cam::g_launches);
    return 0;
}
