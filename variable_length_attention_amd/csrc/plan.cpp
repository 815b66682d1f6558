// Host-side planning of a rank's work (no device code): front/back chunk pairing of a long
// sequence over a ring, HDP sharding of a global batch over a pool of ranks, and the balance
// scheduler.  Research digest "ByteScale: Communication-Efficient Scaling of LLM Training with
// a 2048K Context Length on 16384 GPUs": §3.1 and Figure 2 (HDP pool, ceil(s/C) ranks per long
// sequence, best-fit packing of the short ones), §3.4 and Figure 4 (balance scheduler), §4
// (2N chunks handed out in front/back pairs).
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "hdp_attn.h"

extern "C" {

int hdp_pair_chunks(int64_t s, int32_t n_ranks, int32_t rank, int64_t* offsets, int64_t* lengths) {
    if (s < 0 || n_ranks <= 0 || rank < 0 || rank >= n_ranks || !offsets || !lengths)
        return HDP_ERR_INVALID_ARG;
    const int64_t n2 = 2 * (int64_t)n_ranks;
    // chunk c = [bound(c), bound(c+1)); c <= 2N and s < 2^63, so c * s fits in 128 bits and the
    // quotient, at most s, fits in int64
    auto bound = [&](int64_t c) { return (int64_t)((__int128)c * s / n2); };
    const int64_t c[2] = {rank, n2 - 1 - rank};
    for (int i = 0; i < 2; ++i) {
        offsets[i] = bound(c[i]);
        lengths[i] = bound(c[i] + 1) - offsets[i];
    }
    return HDP_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// HDP sharding of one global batch over a pool of ranks of capacity C tokens (digest §3.1,
// Figure 2).  Units are what one rank holds for one round:
//   * a sequence longer than C gets a ring of ceil(s / C) units; ring unit r holds slice r of
//     ceil(s/C) near-equal contiguous slices, or, with pair != 0, the front/back chunk pair r of
//     2N chunks (hdp_pair_chunks);
//   * shorter sequences are packed by best fit into units of at most C tokens.
// Order: rings by decreasing length (ties: lower index first), then the packed units in the
// order they were opened; short sequences are placed by decreasing length.  With the pages'
// example (32K, 16K, 8K, 4K, 4K at C = 8K) this is exactly Figure 2(b): ranks 0-3 hold the 32K
// ring, 4-5 the 16K ring, 6 the 8K sequence and 7 the two 4K ones.
// ---------------------------------------------------------------------------------------------
extern "C" int hdp_plan_shard(const int64_t* lens, int32_t n_seq, int64_t C, int32_t pair,
                              int32_t max_units, int32_t max_pieces, int32_t* n_units,
                              int32_t* n_pieces, int32_t* unit_first_piece, int32_t* unit_ring,
                              int32_t* piece_seq, int64_t* piece_off, int64_t* piece_len) {
    if (n_seq < 0 || C <= 0 || !n_units || !n_pieces || (n_seq > 0 && !lens)) return HDP_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n_seq; ++i)
        if (lens[i] < 0) return HDP_ERR_INVALID_ARG;
    std::vector<int32_t> order(n_seq);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return lens[a] > lens[b]; });

    struct Unit { int32_t ring; std::vector<int32_t> seqs; std::vector<std::pair<int64_t, int64_t>> span; int64_t used; };
    std::vector<Unit> units;
    // rings
    for (int32_t i : order) {
        const int64_t s = lens[i];
        if (s <= C) continue;
        const int64_t N = (s + C - 1) / C;
        if (N > INT32_MAX) return HDP_ERR_OVERFLOW;
        for (int64_t r = 0; r < N; ++r) {
            Unit u{i, {}, {}, 0};
            if (pair) {
                int64_t off[2], len[2];
                if (int st = hdp_pair_chunks(s, (int32_t)N, (int32_t)r, off, len)) return st;
                for (int h = 0; h < 2; ++h) { u.seqs.push_back(i); u.span.push_back({off[h], len[h]}); }
            } else {
                const int64_t a = (int64_t)((__int128)r * s / N), b = (int64_t)((__int128)(r + 1) * s / N);
                u.seqs.push_back(i);
                u.span.push_back({a, b - a});
            }
            units.push_back(std::move(u));
        }
    }
    // best fit of the short sequences
    const size_t first_packed = units.size();
    for (int32_t i : order) {
        const int64_t s = lens[i];
        if (s > C || s == 0) continue;
        size_t best = units.size();
        for (size_t j = first_packed; j < units.size(); ++j) {
            const int64_t room = C - units[j].used;
            if (room >= s && (best == units.size() || room < C - units[best].used)) best = j;
        }
        if (best == units.size()) {
            units.push_back(Unit{-1, {}, {}, 0});
            best = units.size() - 1;
        }
        units[best].seqs.push_back(i);
        units[best].span.push_back({0, s});
        units[best].used += s;
    }
    int64_t pieces = 0;
    for (const Unit& u : units) pieces += (int64_t)u.seqs.size();
    if ((int64_t)units.size() > INT32_MAX || pieces > INT32_MAX) return HDP_ERR_OVERFLOW;
    *n_units = (int32_t)units.size();
    *n_pieces = (int32_t)pieces;
    if ((int64_t)units.size() > max_units || pieces > max_pieces) return HDP_ERR_OVERFLOW;
    if (!unit_first_piece || !unit_ring || (pieces > 0 && (!piece_seq || !piece_off || !piece_len)))
        return HDP_ERR_INVALID_ARG;
    int32_t p = 0;
    for (size_t j = 0; j < units.size(); ++j) {
        unit_first_piece[j] = p;
        unit_ring[j] = units[j].ring;
        for (size_t t = 0; t < units[j].seqs.size(); ++t, ++p) {
            piece_seq[p] = units[j].seqs[t];
            piece_off[p] = units[j].span[t].first;
            piece_len[p] = units[j].span[t].second;
        }
    }
    unit_first_piece[units.size()] = p;
    return HDP_OK;
}

// Attention FLOPs of each unit of a plan (pass as hdp_seq_flops): a packed unit costs its
// sequences' hdp_seq_flops; a ring unit costs its query pieces against every piece of its ring
// (hdp_chunk_flops, causal), i.e. its share of the ring's work.
extern "C" int hdp_plan_unit_flops(const int64_t* lens, int32_t n_seq, int32_t n_units,
                                   const int32_t* unit_first_piece, const int32_t* unit_ring,
                                   const int32_t* piece_seq, const int64_t* piece_off,
                                   const int64_t* piece_len, int32_t H, int32_t D, int32_t pass,
                                   uint64_t* cost) {
    if (n_units < 0 || !cost || (n_units > 0 && (!unit_first_piece || !unit_ring))) return HDP_ERR_INVALID_ARG;
    for (int32_t j = 0; j < n_units; ++j) {
        unsigned __int128 acc = 0;
        for (int32_t p = unit_first_piece[j]; p < unit_first_piece[j + 1]; ++p) {
            const int32_t i = piece_seq[p];
            if (i < 0 || i >= n_seq) return HDP_ERR_INVALID_ARG;
            if (unit_ring[j] < 0) {
                acc += hdp_seq_flops(lens[i], H, D, 1, pass);
                continue;
            }
            // every piece of the same ring (units are listed ring by ring)
            for (int32_t k = 0; k < n_units; ++k) {
                if (unit_ring[k] != unit_ring[j]) continue;
                for (int32_t t = unit_first_piece[k]; t < unit_first_piece[k + 1]; ++t) {
                    if (piece_len[p] > INT32_MAX || piece_len[t] > INT32_MAX) return HDP_ERR_OVERFLOW;
                    acc += hdp_chunk_flops((int32_t)piece_len[p], (int32_t)piece_len[t], piece_off[p],
                                           piece_off[t], 1, H, D, pass);
                }
            }
        }
        cost[j] = acc > (unsigned __int128)UINT64_MAX ? UINT64_MAX : (uint64_t)acc;
    }
    return HDP_OK;
}

// ---------------------------------------------------------------------------------------------
// Balance scheduler, DP-Balance (digest §3.4 and Figure 4): units hold equal tokens but unequal
// attention work, so ranks run different numbers of them.  The pages describe it in prose only
// ("sort by length into buckets of about equal FLOPs, then give work to every rank that trails
// the slowest one by more than delta; DP-Balance takes from the first bucket").  Our reading:
//   1. items are packed units and whole rings (a ring of w units runs on w distinct ranks at
//      once), sorted by per-rank cost, decreasing (cost = the unit's FLOPs, ring: its largest
//      unit's);
//   2. the sorted list is cut into n_ranks buckets of about equal total FLOPs;
//   3. repeat: the ranks whose load trails the most loaded rank by more than delta (all ranks,
//      when none does) each take, least loaded first, the next item of the first non-empty
//      bucket; a ring takes the w least loaded ranks of that set, or of all ranks if the set is
//      smaller than w.
// unit_rank[j] receives the rank of unit j, rank_load[r] the sum of its units' costs.
// ---------------------------------------------------------------------------------------------
extern "C" int hdp_plan_balance(const uint64_t* cost, const int32_t* unit_ring, int32_t n_units,
                                int32_t n_ranks, uint64_t delta, int32_t* unit_rank,
                                uint64_t* rank_load) {
    if (n_units < 0 || n_ranks <= 0 || !rank_load || (n_units > 0 && (!cost || !unit_ring || !unit_rank)))
        return HDP_ERR_INVALID_ARG;
    struct Item { std::vector<int32_t> units; uint64_t per_rank; };
    std::vector<Item> items;
    for (int32_t j = 0; j < n_units; ++j) {
        if (unit_ring[j] >= 0 && j > 0 && unit_ring[j - 1] == unit_ring[j]) {
            items.back().units.push_back(j);
            items.back().per_rank = std::max(items.back().per_rank, cost[j]);
        } else {
            items.push_back(Item{{j}, cost[j]});
        }
    }
    for (const Item& it : items)
        if ((int64_t)it.units.size() > n_ranks) return HDP_ERR_INVALID_ARG;   // ring wider than the pool
    std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.per_rank > b.per_rank; });
    // buckets of about equal total FLOPs over the sorted items
    unsigned __int128 total = 0;
    for (const Item& it : items) total += (unsigned __int128)it.per_rank * it.units.size();
    std::vector<std::vector<size_t>> buckets(n_ranks);
    {
        unsigned __int128 run = 0;
        for (size_t i = 0; i < items.size(); ++i) {
            const unsigned __int128 w = (unsigned __int128)items[i].per_rank * items[i].units.size();
            size_t b = total == 0 ? 0 : (size_t)((run * (unsigned)n_ranks) / total);
            if (b >= (size_t)n_ranks) b = n_ranks - 1;
            buckets[b].push_back(i);
            run += w;
        }
    }
    std::vector<unsigned __int128> load(n_ranks, 0);
    size_t bi = 0, bj = 0, placed = 0;
    auto next_item = [&]() -> long {
        while (bi < buckets.size() && bj >= buckets[bi].size()) { ++bi; bj = 0; }
        if (bi >= buckets.size()) return -1;
        return (long)buckets[bi][bj];
    };
    while (placed < items.size()) {
        unsigned __int128 top = 0;
        for (auto x : load) top = std::max(top, x);
        std::vector<int32_t> trail;
        for (int32_t r = 0; r < n_ranks; ++r)
            if (top - load[r] > delta) trail.push_back(r);
        if (trail.empty()) {
            trail.resize(n_ranks);
            std::iota(trail.begin(), trail.end(), 0);
        }
        std::stable_sort(trail.begin(), trail.end(), [&](int32_t a, int32_t b) { return load[a] < load[b]; });
        std::vector<char> taken(n_ranks, 0);
        for (size_t t = 0; t < trail.size() && placed < items.size(); ++t) {
            if (taken[trail[t]]) continue;
            const long ii = next_item();
            if (ii < 0) break;
            const Item& it = items[ii];
            std::vector<int32_t> ranks;
            for (size_t u = t; u < trail.size() && ranks.size() < it.units.size(); ++u)
                if (!taken[trail[u]]) ranks.push_back(trail[u]);
            if (ranks.size() < it.units.size()) {       // not enough trailing ranks: least loaded overall
                std::vector<int32_t> all(n_ranks);
                std::iota(all.begin(), all.end(), 0);
                std::stable_sort(all.begin(), all.end(), [&](int32_t a, int32_t b) { return load[a] < load[b]; });
                ranks.clear();
                for (int32_t r : all)
                    if (ranks.size() < it.units.size() && !taken[r]) ranks.push_back(r);
                if (ranks.size() < it.units.size()) break;   // next round
            }
            for (size_t u = 0; u < it.units.size(); ++u) {
                unit_rank[it.units[u]] = ranks[u];
                load[ranks[u]] += cost[it.units[u]];
                taken[ranks[u]] = 1;
            }
            ++bj;
            ++placed;
        }
    }
    for (int32_t r = 0; r < n_ranks; ++r) rank_load[r] = load[r] > (unsigned __int128)UINT64_MAX ? UINT64_MAX : (uint64_t)load[r];
    return HDP_OK;
}
