// thd_planner.cpp -- host-side THD layout planner for context parallelism over
// packed sequences (cuLA PR "feat(distributed): add packed hybrid runtime and
// THD planner", description and planner tests).  What the plan must do: keep
// each rank's work even, both the part that grows with its token count and
// the part that grows with causal position, for any packed batch; leave a
// short sample on one rank; deal long sequences out in a direction that flips
// from rank to rank; try several grids and keep the plain contiguous layout
// as a candidate; give every rank the same number of aligned blocks; return
// the same span list for the same input.  Input checks follow the PR's
// planner tests.
//
// The page does not print the steps; this is the reading implemented:
//   - capacity: rank r holds exactly floor((r+1)N/W) - floor(rN/W) of the
//     N blocks (balanced shards, any W);
//   - cost of a token at position k of its sequence: token_weight +
//     causal_weight * (k + 1); a rank's cost sums its tokens' costs;
//   - candidate 0 is the contiguous layout; candidate g = 1..6 places the
//     short samples whole (costliest first, cheapest rank with room), deals
//     each long sequence's W * 2^(g-1) chunks along a snake whose direction
//     alternates per round and per long sequence, moves blocks of overfull
//     ranks (the top of the highest long span or the bottom of the lowest,
//     whichever suits the pair) to the cheapest ranks with room, lays any
//     short that fitted nowhere into the remaining room, and finally
//     exchanges equal block counts between the costliest and the cheapest
//     rank (high positions for low) while that lowers their larger cost;
//   - the least maximum rank cost wins (ties: fewer spans, lower candidate),
//     candidates over max_chunks_per_rank spans per rank excepted.
// Host code only: no HIP call.  The span tables it writes drive the planned
// varlen relayout (ulysses_seq_to_head_spans / ulysses_head_to_seq_spans).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "cam_internal.h"

// Costs are compared for equality between candidates: keep every product and
// sum separately rounded (no fused multiply-add), so a plan is reproducible.
#pragma clang fp contract(off)

namespace cam {
namespace {

struct Span {
    int64_t seq;
    int64_t lo, hi;  // blocks [lo, hi) of the sequence
    int64_t rank;
};

struct Batch {
    std::vector<int64_t> blocks;  // per sequence
    std::vector<int64_t> cap;     // per rank, blocks
    int64_t W = 0, b = 0, min_split = 0;
    double wt = 0, wc = 0;
    bool is_long(int64_t i) const { return blocks[i] >= 2 && blocks[i] * b >= min_split; }
};

// sum of (k + 1) for k in [0, n)
inline int64_t prefix_work(int64_t n) { return n * (n + 1) / 2; }

struct Ledger {
    const Batch& B;
    std::vector<int64_t> held, causal;  // per rank: blocks, sum of (k + 1)
    explicit Ledger(const Batch& batch) : B(batch), held(batch.W, 0), causal(batch.W, 0) {}
    double cost(int64_t r) const
    {
        const double tokens_part = B.wt * double(held[r] * B.b);
        const double causal_part = B.wc * double(causal[r]);
        return tokens_part + causal_part;
    }
    void add(int64_t r, int64_t lo, int64_t hi, int64_t sign)
    {
        held[r] += sign * (hi - lo);
        causal[r] += sign * (prefix_work(hi * B.b) - prefix_work(lo * B.b));
    }
    int64_t room(int64_t r) const { return B.cap[r] - held[r]; }
    // cheapest rank with at least `need` blocks of room; -1 when none
    int64_t cheapest(int64_t need) const
    {
        int64_t pick = -1;
        for (int64_t r = 0; r < B.W; ++r) {
            if (room(r) < need)
                continue;
            if (pick < 0 || cost(r) < cost(pick))
                pick = r;
        }
        return pick;
    }
};

std::vector<Span> contiguous(const Batch& B)
{
    std::vector<Span> out;
    int64_t N = 0;
    for (int64_t n : B.blocks)
        N += n;
    int64_t first = 0;  // global block of the sequence's first block
    for (int64_t i = 0; i < int64_t(B.blocks.size()); ++i) {
        const int64_t last = first + B.blocks[i];
        for (int64_t r = 0; r < B.W; ++r) {
            const int64_t lo = std::max(r * N / B.W, first), hi = std::min((r + 1) * N / B.W, last);
            if (lo < hi)
                out.push_back({i, lo - first, hi - first, r});
        }
        first = last;
    }
    return out;
}

std::vector<Span> grid(const Batch& B, int g)
{
    const int64_t nseq = int64_t(B.blocks.size());
    const int64_t chunks = B.W << (g - 1);
    Ledger led(B);
    std::vector<Span> out;

    // short samples, whole, costliest first (stable: batch order on ties)
    std::vector<int64_t> shorts;
    for (int64_t i = 0; i < nseq; ++i)
        if (B.blocks[i] > 0 && !B.is_long(i))
            shorts.push_back(i);
    auto whole_cost = [&](int64_t i) {
        const double tokens_part = B.wt * double(B.blocks[i] * B.b);
        const double causal_part = B.wc * double(prefix_work(B.blocks[i] * B.b));
        return tokens_part + causal_part;
    };
    std::stable_sort(shorts.begin(), shorts.end(),
                     [&](int64_t x, int64_t y) { return whole_cost(x) > whole_cost(y); });
    std::vector<int64_t> unplaced;
    for (int64_t i : shorts) {
        const int64_t r = led.cheapest(B.blocks[i]);
        if (r < 0) {
            unplaced.push_back(i);
        } else {
            out.push_back({i, 0, B.blocks[i], r});
            led.add(r, 0, B.blocks[i], +1);
        }
    }

    // long sequences: snake over the ranks, direction flipping per round and
    // per long sequence
    int64_t nth_long = 0;
    for (int64_t i = 0; i < nseq; ++i) {
        if (!B.is_long(i))
            continue;
        const int64_t n = B.blocks[i];
        const int64_t m = std::min(n, chunks);
        for (int64_t c = 0; c < m; ++c) {
            const int64_t lo = c * n / m, hi = (c + 1) * n / m;
            const int64_t step = c % B.W;
            const bool forward = ((c / B.W) + nth_long) % 2 == 0;
            const int64_t r = forward ? step : B.W - 1 - step;
            out.push_back({i, lo, hi, r});
            led.add(r, lo, hi, +1);
        }
        ++nth_long;
    }

    // the long span of rank r ending highest (ties: later sequence) and the
    // one starting lowest (ties: earlier sequence)
    auto highest = [&](int64_t r) {
        Span* pick = nullptr;
        for (Span& s : out)
            if (s.rank == r && s.lo < s.hi && B.is_long(s.seq) &&
                (!pick || s.hi > pick->hi || (s.hi == pick->hi && s.seq > pick->seq)))
                pick = &s;
        return pick;
    };
    auto lowest = [&](int64_t r) {
        Span* pick = nullptr;
        for (Span& s : out)
            if (s.rank == r && s.lo < s.hi && B.is_long(s.seq) &&
                (!pick || s.lo < pick->lo || (s.lo == pick->lo && s.seq < pick->seq)))
                pick = &s;
        return pick;
    };
    // larger cost of ranks x and y after moving blocks [lo, hi) from x to y
    auto after_move = [&](int64_t x, int64_t y, int64_t lo, int64_t hi) {
        led.add(x, lo, hi, -1);
        led.add(y, lo, hi, +1);
        const double worst = std::max(led.cost(x), led.cost(y));
        led.add(y, lo, hi, -1);
        led.add(x, lo, hi, +1);
        return worst;
    };

    // token rebalancing: an overfull rank sheds blocks from the top of its
    // highest long span or the bottom of its lowest, whichever suits the pair
    for (;;) {
        int64_t over = -1;
        for (int64_t r = 0; r < B.W && over < 0; ++r)
            if (led.room(r) < 0)
                over = r;
        if (over < 0)
            break;
        Span* top = highest(over);
        Span* bottom = lowest(over);
        const int64_t to = led.cheapest(1);
        const int64_t want = std::min(-led.room(over), led.room(to));
        const int64_t n_top = std::min(want, top->hi - top->lo), n_bottom = std::min(want, bottom->hi - bottom->lo);
        const double via_top = after_move(over, to, top->hi - n_top, top->hi);
        const double via_bottom = after_move(over, to, bottom->lo, bottom->lo + n_bottom);
        Span piece;
        if (via_bottom < via_top) {
            piece = {bottom->seq, bottom->lo, bottom->lo + n_bottom, to};
            bottom->lo += n_bottom;
        } else {
            piece = {top->seq, top->hi - n_top, top->hi, to};
            top->hi -= n_top;
        }
        led.add(over, piece.lo, piece.hi, -1);
        out.push_back(piece);
        led.add(to, piece.lo, piece.hi, +1);
    }

    // shorts that fitted nowhere whole fill the remaining room
    for (int64_t i : unplaced) {
        for (int64_t lo = 0; lo < B.blocks[i];) {
            const int64_t r = led.cheapest(1);
            const int64_t hi = std::min(B.blocks[i], lo + led.room(r));
            out.push_back({i, lo, hi, r});
            led.add(r, lo, hi, +1);
            lo = hi;
        }
    }
    // exchanges between the costliest and the cheapest rank: equal block
    // counts, the top of the costliest rank's highest long span for the bottom
    // of the cheapest rank's lowest, while that lowers the pair's larger cost
    for (int64_t round = 0; round < 4 * B.W; ++round) {
        int64_t hot = 0, cold = 0;
        for (int64_t r = 1; r < B.W; ++r) {
            if (led.cost(r) > led.cost(hot))
                hot = r;
            if (led.cost(r) < led.cost(cold))
                cold = r;
        }
        if (hot == cold)
            break;
        Span* give = highest(hot);
        Span* take = lowest(cold);
        if (!give || !take)
            break;
        double best = std::max(led.cost(hot), led.cost(cold));
        int64_t best_n = 0;
        const int64_t limit = std::min(give->hi - give->lo, take->hi - take->lo);
        for (int64_t n = 1; n <= limit; ++n) {
            led.add(hot, give->hi - n, give->hi, -1);
            led.add(cold, give->hi - n, give->hi, +1);
            const double worst = after_move(cold, hot, take->lo, take->lo + n);
            led.add(cold, give->hi - n, give->hi, -1);
            led.add(hot, give->hi - n, give->hi, +1);
            if (worst < best) {
                best = worst;
                best_n = n;
            }
        }
        if (best_n == 0)
            break;
        const Span down{give->seq, give->hi - best_n, give->hi, cold};
        const Span up{take->seq, take->lo, take->lo + best_n, hot};
        give->hi -= best_n;
        take->lo += best_n;
        led.add(hot, down.lo, down.hi, -1);
        led.add(cold, down.lo, down.hi, +1);
        led.add(cold, up.lo, up.hi, -1);
        led.add(hot, up.lo, up.hi, +1);
        out.push_back(down);
        out.push_back(up);
    }
    out.erase(std::remove_if(out.begin(), out.end(), [](const Span& s) { return s.lo >= s.hi; }), out.end());
    return out;
}

// packed order; spans of one sequence that meet on one rank become one
void canonical(std::vector<Span>& v)
{
    std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) {
        return x.seq != y.seq ? x.seq < y.seq : x.lo < y.lo;
    });
    std::vector<Span> merged;
    for (const Span& s : v) {
        if (!merged.empty() && merged.back().seq == s.seq && merged.back().rank == s.rank && merged.back().hi == s.lo)
            merged.back().hi = s.hi;
        else
            merged.push_back(s);
    }
    v.swap(merged);
}

}  // namespace
}  // namespace cam

using namespace cam;

extern "C" cam_status thd_plan(const int32_t* cu_seqlens, int64_t nseq, int64_t world_size,
                               const cam_thd_planner_config* cfg, int64_t max_spans, int32_t* span_start,
                               int32_t* span_rank, int32_t* span_local, int64_t* rank_off, double* rank_cost,
                               int64_t* n_spans, int32_t* chosen)
{
    const char* op = "thd_plan";
    clear_error();
    if (!cu_seqlens || !cfg || !n_spans || !chosen)
        return set_error(CAM_ERR_NULL, "%s: cu_seqlens, cfg, n_spans and chosen must be non-null", op);
    const int64_t b = cfg->block_size;
    if (world_size < 1)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: world_size must be >= 1", op);
    if (b < 1 || cfg->min_split_tokens < 1 || cfg->max_chunks_per_rank < 1)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: block_size, min_split_tokens and max_chunks_per_rank must be "
                                              "positive", op);
    if (cfg->min_split_tokens % b != 0)
        return set_error(CAM_ERR_ALIGNMENT, "%s: min_split_tokens must be a multiple of block_size", op);
    if (!std::isfinite(cfg->token_weight) || !std::isfinite(cfg->causal_weight) || cfg->token_weight < 0 ||
        cfg->causal_weight < 0 || (cfg->token_weight == 0 && cfg->causal_weight == 0))
        return set_error(CAM_ERR_UNSUPPORTED, "%s: cost weights must be finite, non-negative and not both zero", op);
    if (cfg->mode != 0 && cfg->mode != 1)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: mode must be 0 (planned) or 1 (contiguous)", op);
    if (nseq < 0 || cu_seqlens[0] != 0)
        return set_error(CAM_ERR_SHAPE, "%s: cu_seqlens must start at 0 and nseq be >= 0", op);
    Batch B;
    B.W = world_size;
    B.b = b;
    B.min_split = cfg->min_split_tokens;
    B.wt = cfg->token_weight;
    B.wc = cfg->causal_weight;
    int64_t N = 0;
    for (int64_t i = 0; i < nseq; ++i) {
        const int64_t len = int64_t(cu_seqlens[i + 1]) - cu_seqlens[i];
        if (len < 0)
            return set_error(CAM_ERR_SHAPE, "%s: cu_seqlens must be non-decreasing", op);
        if (len % b != 0)
            return set_error(CAM_ERR_ALIGNMENT, "%s: sequence %lld has %lld tokens, not a multiple of block_size %lld",
                             op, (long long)i, (long long)len, (long long)b);
        B.blocks.push_back(len / b);
        N += len / b;
    }
    if (N < world_size)
        return set_error(CAM_ERR_SHAPE, "%s: %lld aligned blocks for %lld ranks", op, (long long)N,
                         (long long)world_size);
    for (int64_t r = 0; r < world_size; ++r)
        B.cap.push_back((r + 1) * N / world_size - r * N / world_size);

    std::vector<Span> best;
    double best_max = 0;
    int best_g = -1;
    const int last = cfg->mode == 1 ? 0 : 6;
    for (int g = 0; g <= last; ++g) {
        std::vector<Span> cand = g == 0 ? contiguous(B) : grid(B, g);
        canonical(cand);
        Ledger led(B);
        std::vector<int64_t> count(world_size, 0);
        for (const Span& s : cand) {
            led.add(s.rank, s.lo, s.hi, +1);
            ++count[s.rank];
        }
        double worst = led.cost(0);
        for (int64_t r = 1; r < world_size; ++r)
            worst = std::max(worst, led.cost(r));
        if (g > 0 && *std::max_element(count.begin(), count.end()) > cfg->max_chunks_per_rank)
            continue;
        if (best_g < 0 || worst < best_max || (worst == best_max && cand.size() < best.size())) {
            best.swap(cand);
            best_max = worst;
            best_g = g;
        }
    }
    *n_spans = int64_t(best.size());
    if (int64_t(best.size()) > max_spans)
        return set_error(CAM_ERR_SHAPE, "%s: the plan has %lld spans, the tables hold %lld", op,
                         (long long)best.size(), (long long)max_spans);
    if (!span_start || !span_rank || !span_local || !rank_off || !rank_cost)
        return set_error(CAM_ERR_NULL, "%s: output tables must be non-null", op);
    Ledger led(B);
    std::vector<int64_t> next(world_size, 0);  // next local row per rank
    for (size_t k = 0; k < best.size(); ++k) {
        const Span& s = best[k];
        span_start[k] = int32_t(cu_seqlens[s.seq] + s.lo * b);
        span_rank[k] = int32_t(s.rank);
        span_local[k] = int32_t(next[s.rank]);
        next[s.rank] += (s.hi - s.lo) * b;
        led.add(s.rank, s.lo, s.hi, +1);
    }
    // every rank must hold exactly its capacity: the relayouts place rank r's
    // slab at rank_off[r] and would leave rows unwritten otherwise
    for (int64_t r = 0; r < world_size; ++r)
        if (next[r] != B.cap[r] * b)
            return set_error(CAM_ERR_SHAPE, "%s: rank %lld holds %lld tokens, its capacity is %lld", op,
                             (long long)r, (long long)next[r], (long long)(B.cap[r] * b));
    span_start[best.size()] = cu_seqlens[nseq];
    rank_off[0] = 0;
    for (int64_t r = 0; r < world_size; ++r) {
        rank_off[r + 1] = rank_off[r] + B.cap[r] * b;
        rank_cost[r] = led.cost(r);
    }
    *chosen = best_g;
    return CAM_OK;
}

// Smallest position of each sequence that each rank holds, from a plan's
// span tables (the causal rule of the planned combine: partial p of a token
// at position k of sequence i is admitted iff first_pos[p][i] <= k).
extern "C" cam_status thd_plan_first_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t world_size,
                                               const int32_t* span_start, const int32_t* span_rank,
                                               int64_t n_spans, int32_t* first_pos)
{
    const char* op = "thd_plan_first_positions";
    clear_error();
    if (nseq < 0 || world_size < 1 || n_spans < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need nseq >= 0, world_size >= 1, n_spans >= 0", op);
    if (!cu_seqlens || !first_pos || (n_spans > 0 && (!span_start || !span_rank)))
        return set_error(CAM_ERR_NULL, "%s: null table", op);
    std::fill(first_pos, first_pos + world_size * nseq, INT32_MAX);
    for (int64_t s = 0; s < n_spans; ++s) {
        const int32_t t = span_start[s];
        // the sequence whose token range holds the span's first token
        const int32_t* hit = std::upper_bound(cu_seqlens, cu_seqlens + nseq + 1, t);
        const int64_t i = int64_t(hit - cu_seqlens) - 1;
        const int64_t r = span_rank[s];
        if (i < 0 || i >= nseq || r < 0 || r >= world_size)
            return set_error(CAM_ERR_SHAPE, "%s: span %lld lies outside the batch or the ranks", op, (long long)s);
        int32_t& f = first_pos[r * nseq + i];
        f = std::min(f, int32_t(t - cu_seqlens[i]));
    }
    return CAM_OK;
}

