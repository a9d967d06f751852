// Host side of the compute waves' work lists: for one launch of the pass kernel, every
// compute wave's steps in order, each with the address offset of its two chunks, the LDS
// offset of its activations and what the wave does around it (close units, enter a
// stage).  Built once per shape on the host, where every address is checked against its
// matrix, and read by the waves with scalar loads.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "vq_internal.h"

namespace vq {

// One entry: x = byte offset of the step's first chunk from its matrix; y = flags:
constexpr uint32_t ST_XOFF_MASK = 0x3fffu;   // bits 0..13: LDS activation offset / 16
constexpr int ST_CLOSE_SHIFT = 14;           // bits 14..21: units to close before the step
constexpr uint32_t ST_CLOSE_MAX = 255u;
constexpr uint32_t ST_OPEN = 1u << 22;       // first step of the wave in its stage
constexpr uint32_t ST_VALID = 1u << 23;      // a step with chunks (else: closes only)
constexpr int ST_STAGE_SHIFT = 24;           // bits 24..30: stage - s_begin of the launch (of the
                                             // chunk's matrix, also without ST_VALID)
constexpr uint32_t ST_END = 1u << 31;        // the wave's last entry (closes only) and padding
constexpr int ST_ROUND = 4;                  // entries a wave reads per round

struct StepTable {
    std::vector<uint32_t> ent;     // pairs (offset, flags)
    std::vector<uint32_t> start;   // per workgroup and compute wave: index of its first pair
    void put_ent(uint32_t v) { ent.push_back(v); }
    void put_start(uint32_t v) { start.push_back(v); }
    size_t n_ent() const { return ent.size(); }
    size_t n_start() const { return start.size(); }
    bool ok() const { return true; }
};

// The same in caller-owned fixed storage (no allocation); ok() turns false once full.
struct FixedStepTable {
    uint32_t* ent;
    size_t ent_cap, ne = 0;
    uint32_t* start;
    size_t start_cap, ns = 0;
    bool full = false;
    void put_ent(uint32_t v) {
        if (ne < ent_cap) ent[ne++] = v;
        else full = true;
    }
    void put_start(uint32_t v) {
        if (ns < start_cap) start[ns++] = v;
        else full = true;
    }
    size_t n_ent() const { return ne; }
    size_t n_start() const { return ns; }
    bool ok() const { return !full; }
};

namespace steps {

// Position of step c of a stage: window, tile, step inside the window, steps of that window.
struct Pos {
    int w, t, i, gl;
};
inline Pos locate(const KindPlan& P, long c) {
    Pos p;
    const long span = (long)P.T * P.gw;
    const long lastb = (long)(P.nwin - 1) * span;
    if (c < lastb) {
        p.w = (int)(c / span);
        const long r = c - p.w * span;
        p.t = (int)(r / P.gw);
        p.i = (int)(r - (long)p.t * P.gw);
        p.gl = P.gw;
    } else {
        p.w = P.nwin - 1;
        const long r = c - lastb;
        p.t = (int)(r / P.glast);
        p.i = (int)(r - (long)p.t * P.glast);
        p.gl = P.glast;
    }
    return p;
}

// A workgroup's steps of a stage in processing order: segment A (the tail of its range when
// that unit continues in the next workgroup's range), then segment B (the rest, in order);
// units in processing order: A's unit, then B's units in increasing flat index.
struct Seq {
    long lo, hi, a0;
    int n, lenA, nU, uA, uB0, wlo;
};
inline Seq seq_of(const KindPlan& P, int w) {
    Seq q{};
    if (w >= P.nwe) return q;
    q.lo = (long)w * P.q + std::min(w, P.r);
    q.hi = q.lo + P.q + (w < P.r ? 1 : 0);
    q.n = (int)(q.hi - q.lo);
    const Pos pl = locate(P, q.hi - 1);
    const long ustart = q.hi - 1 - pl.i;
    q.a0 = q.hi;
    if (ustart + pl.gl > q.hi) q.a0 = std::max(ustart, q.lo);
    q.lenA = (int)(q.hi - q.a0);
    const Pos p0 = locate(P, q.lo);
    q.wlo = p0.w;
    q.uB0 = p0.w * P.T + p0.t;
    q.uA = pl.w * P.T + pl.t;
    int nb = 0;
    if (q.a0 - q.lo > 0) {
        const Pos pb = locate(P, q.a0 - 1);
        nb = pb.w * P.T + pb.t - q.uB0 + 1;
    }
    q.nU = (q.lenA > 0 ? 1 : 0) + nb;
    return q;
}
inline long seq_step(const Seq& q, int k) { return k < q.lenA ? q.a0 + k : q.lo + (k - q.lenA); }
inline int unit_pos(const Seq& q, int U) {
    if (q.lenA > 0) return U == q.uA ? 0 : 1 + (U - q.uB0);
    return U - q.uB0;
}

}  // namespace steps

// How a stage's steps are dealt to the compute waves: step k goes to wave deal()[k % n].
// Dealt in equal shares, the waves of a SIMD do not finish together: wave i sits on SIMD
// i % 4 (the conductor on SIMD 3), the SIMD issues for its older waves first, and at K <= 8
// the last wave of each SIMD finished its steps ~45% later than the first, alone on its
// SIMD by then.  The weighted deal gives wave i kWaveWeight[i] steps of every 86, each step
// to the wave whose share would then be least ahead (ties to the lower wave), so that the
// steps of a wave are spread evenly.  The weights were chosen by timing the 27B pass at
// K = 1 and 8 over several tables: the youngest waves (8..10) do best with clearly less than
// their rate share (they also start each stage late), waves 4..7 with about an equal one.
constexpr int kWaveWeight[FLOW_NCW] = {10, 10, 10, 9, 9, 9, 9, 8, 6, 6, 6};
struct Deal {
    uint8_t wave[128];
    int n;
};
inline Deal make_deal(bool weighted) {
    Deal d{};
    int wsum = 0;
    for (int i = 0; i < FLOW_NCW; ++i) wsum += weighted ? kWaveWeight[i] : 1;
    int cnt[FLOW_NCW] = {};
    d.n = wsum;
    for (int k = 0; k < wsum; ++k) {
        int best = 0;
        for (int i = 1; i < FLOW_NCW; ++i) {
            // (cnt + 1) / weight, compared exactly
            const long wi = weighted ? kWaveWeight[i] : 1, wb = weighted ? kWaveWeight[best] : 1;
            if ((long)(cnt[i] + 1) * wb < (long)(cnt[best] + 1) * wi) best = i;
        }
        d.wave[k] = (uint8_t)best;
        ++cnt[best];
    }
    return d;
}
inline const Deal& deal(bool weighted) {
    static const Deal w = make_deal(true), e = make_deal(false);
    return weighted ? w : e;
}
static_assert(10 + 10 + 10 + 9 + 9 + 9 + 9 + 8 + 6 + 6 + 6 <= 128, "the pattern fits");

// The kind of launch stage s (the pass: 4 per layer, then the lm_head; or one linear map).
inline int stage_kind(int s, int L, bool linear) {
    if (linear) return SK_LIN;
    if (s == 4 * L) return SK_LM;
    return s & 3;
}

// Appends the work lists of one launch (stages [s_begin, s_end), grid nwg) to T.  Returns
// false if an entry would not fit its fields or an address would leave its matrix.
template <class Table>
bool build_steps(Table& T, const KindPlan kp[6], int s_begin, int s_end, int L, bool linear, int nwg, int xoff1,
                 bool weighted) {
    using namespace steps;
    if (s_end - s_begin > 127 || s_end <= s_begin || xoff1 % 16) return false;
    const Deal& dl = deal(weighted);
    Seq seqs[127];
    for (int w = 0; w < nwg; ++w) {
        for (int s = s_begin; s < s_end; ++s)
            seqs[s - s_begin] = seq_of(kp[stage_kind(s, L, linear)], w);
        for (int cw = 0; cw < FLOW_NCW; ++cw) {
            T.put_start((uint32_t)(T.n_ent() / 2));
            const size_t first = T.n_ent();
            uint32_t pending = 0;        // units left behind, not yet closed
            // An entry without chunks still names a chunk (the last valid one, else the first
            // of the launch's first matrix): the waves load every entry's chunks, so that the
            // number of loads in flight is the same in every round.
            uint32_t last_off = 0, last_stage = 0;
            auto emit = [&](uint32_t off, uint32_t flags) {
                while (pending > ST_CLOSE_MAX) {
                    T.put_ent(last_off);
                    T.put_ent((ST_CLOSE_MAX << ST_CLOSE_SHIFT) | (last_stage << ST_STAGE_SHIFT));
                    pending -= ST_CLOSE_MAX;
                }
                if (flags & ST_VALID) {
                    last_off = off;
                    last_stage = (flags >> ST_STAGE_SHIFT) & 127u;
                } else {
                    off = last_off;
                    flags |= last_stage << ST_STAGE_SHIFT;
                }
                T.put_ent(off);
                T.put_ent(flags | (pending << ST_CLOSE_SHIFT));
                pending = 0;
            };
            for (int s = s_begin; s < s_end; ++s) {
                const KindPlan& P = kp[stage_kind(s, L, linear)];
                const Seq& q = seqs[s - s_begin];
                if (q.n == 0) continue;
                const long mat_bytes = (long)P.T * P.G * P.cb;
                int closed = 0;
                bool first = true;
                for (int k = 0; k < q.n; ++k) {
                    if (dl.wave[k % dl.n] != cw) continue;
                    const long c = seq_step(q, k);
                    const Pos p = locate(P, c);
                    const int up = unit_pos(q, p.w * P.T + p.t);
                    if (up < closed || up >= q.nU) return false;
                    pending += (uint32_t)(up - closed);
                    closed = up;
                    const long off = ((long)p.t * P.G + (long)p.w * P.gw + p.i) * P.cb;
                    const long xoff = (long)(p.w - q.wlo) * xoff1 + (long)p.i * 512;
                    if (off < 0 || off + P.cb > mat_bytes || off > 0xffffffffL) return false;
                    if (p.w - q.wlo < 0 || p.w - q.wlo > 1 || xoff % 16 || (xoff >> 4) > (long)ST_XOFF_MASK) return false;
                    if ((long)p.i * 512 + 512 > (long)P.gw * 512) return false;
                    emit((uint32_t)off, (uint32_t)(xoff >> 4) | (first ? ST_OPEN : 0u) | ST_VALID |
                                            ((uint32_t)(s - s_begin) << ST_STAGE_SHIFT));
                    first = false;
                }
                pending += (uint32_t)(q.nU - closed);
            }
            emit(0, ST_END);
            // whole rounds, and two more rounds of padding: the waves read two rounds ahead
            while ((T.n_ent() - first) / 2 % ST_ROUND && T.ok()) emit(0, ST_END);
            for (int i = 0; i < 2 * ST_ROUND; ++i) emit(0, ST_END);
        }
    }
    return T.ok() && T.n_ent() / 2 < (1ul << 32);
}

}  // namespace vq
