// lookback_model.cpp -- a host model of the segment look-back protocol of the
// segmented token-causal forward, for ThreadSanitizer (CPU only, test code).
//
// The state a segment of n tokens hands on is an affine map of the state it
// starts from ([P1] "KV 바인딩 기반 테스트 시간 학습은 사실상 선형
// 어텐션이다", paragraphs on momentum and on associativity once weight
// normalisation is gone; [P2] "In-Place 테스트 시점 학습", paragraph on the
// associative scan):
//     (S, m) -> (S + a m + X, g m + Y),  a = beta + ... + beta^n,  g = beta^n.
// Threads play workgroups.  Thread i belongs to group i % G (G = 8 when the
// heads split evenly into 8 groups, else 1, as the kernel groups workgroups
// by blockIdx % 8) and takes a ticket from its group's counter; ticket t of
// group g runs segment t / per of (head, tile) pair t % per of that group's
// heads (per = nbv / G; heads bh = 8 i + g).  It computes its aggregate (X, Y), publishes it behind a release store of its
// flag (1), walks back over earlier segments with acquire loads (aggregates
// back to the inclusive state of segment s - kChain, or past segment 0 onto
// (S0, M0)), publishes its inclusive state (flag 2) if a later segment reads
// it, and records its start state.  The model checks, over many runs:
//   - every start state equals a single-threaded evaluation of the same walk,
//     bit for bit (the walk has a fixed shape, so timing cannot change it);
//   - it matches the plain sequential chain of segment maps to rounding;
//   - no wait gave up.
// Under -fsanitize=thread, any slot read not ordered after its write by the
// flag's release/acquire pair is reported as a data race.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <thread>
#include <vector>

namespace {

constexpr int kChain = 8;      // as the kernel: segments per link of the inclusive chain
constexpr int kElems = 16;     // state entries per (S, m) block in the model
constexpr long kMaxPolls = 1L << 26;

struct Block {
    float S[kElems], M[kElems];
};

struct Run {
    int nbv, nseg, nvt, groups;
    float beta, a_seg, g_seg;
    std::vector<Block> agg, incl, start;   // [nwg] each
    std::vector<Block> S0;                 // [nbv]
    std::unique_ptr<std::atomic<int>[]> flags, tickets;
    std::atomic<int> error{0};

    Run(int nbv_, int nseg_, int nvt_, float beta_)
        : nbv(nbv_), nseg(nseg_), nvt(nvt_), groups((nbv_ / nvt_) % 8 == 0 ? 8 : 1), beta(beta_) {
        const int nwg = nbv * nseg;
        tickets.reset(new std::atomic<int>[groups]);
        for (int g = 0; g < groups; ++g) tickets[g].store(0, std::memory_order_relaxed);
        agg.resize(nwg);
        incl.resize(nwg);
        start.resize(nwg);
        S0.resize(nbv);
        flags.reset(new std::atomic<int>[nwg]);
        for (int i = 0; i < nwg; ++i) flags[i].store(0, std::memory_order_relaxed);
        const int n = 1024;   // tokens per segment
        const double bn = std::pow((double)beta, n);
        a_seg = (float)(beta * (1.0 - bn) / (1.0 - beta));
        g_seg = (float)bn;
    }
};

// deterministic pseudo-random aggregate of (segment, column pair), in [-1, 1)
float value(int seg, int bv, int e, int which) {
    unsigned x = (unsigned)(seg * 7919 + bv * 104729 + e * 31 + which * 1000003) * 2654435761u;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    return (float)(x & 0xffffff) / (float)(1 << 23) - 1.f;
}

// start state of segment `seg` by the fixed walk, from a read-function
// (blocking in the threaded run, direct in the reference)
template <typename Read>
Block walk(const Run& r, int seg, int bv, Read read) {
    Block T{};   // running map T(S, m) = (S + aT m + XT, gT m + YT), applied at the end
    float aT = 0.f, gT = 1.f;
    bool base = false;
    for (int j = seg - 1; j >= 0 && !base; --j) {
        const bool is_base = (seg - j == kChain);
        const Block& b = read(j, bv, is_base ? 2 : 1);
        for (int e = 0; e < kElems; ++e) {
            T.S[e] += b.S[e] + aT * b.M[e];
            T.M[e] += gT * b.M[e];
        }
        if (is_base) {
            base = true;
        } else {
            aT = r.a_seg + aT * r.g_seg;
            gT = gT * r.g_seg;
        }
    }
    if (!base) {
        const Block& s0 = r.S0[bv];
        for (int e = 0; e < kElems; ++e) {
            T.S[e] += s0.S[e] + aT * s0.M[e];
            T.M[e] += gT * s0.M[e];
        }
    }
    return T;
}

void workgroup(Run* r, int index) {
    const int G = r->groups, grp = index % G;
    const int t = r->tickets[grp].fetch_add(1, std::memory_order_relaxed);
    const int per = r->nbv / G, q = t % per;
    const int seg = t / per, bv = ((q / r->nvt) * G + grp) * r->nvt + q % r->nvt, id = seg * r->nbv + bv;
    const bool last = seg == r->nseg - 1;
    if (!last) {
        Block& a = r->agg[id];
        for (int e = 0; e < kElems; ++e) {
            a.S[e] = value(seg, bv, e, 0);
            a.M[e] = value(seg, bv, e, 1);
        }
        r->flags[id].store(1, std::memory_order_release);
    }
    auto read = [&](int j, int bvj, int want) -> const Block& {
        const int idj = j * r->nbv + bvj;
        long polls = 0;
        while (r->flags[idj].load(std::memory_order_acquire) < want) {
            if (++polls > kMaxPolls) {
                r->error.store(1, std::memory_order_relaxed);
                break;
            }
            std::this_thread::yield();
        }
        return want == 2 ? r->incl[idj] : r->agg[idj];
    };
    const Block st = walk(*r, seg, bv, read);
    r->start[id] = st;
    if (seg + kChain < r->nseg) {
        Block& inc = r->incl[id];
        const Block& a = r->agg[id];
        for (int e = 0; e < kElems; ++e) {
            inc.S[e] = a.S[e] + st.S[e] + r->a_seg * st.M[e];
            inc.M[e] = a.M[e] + r->g_seg * st.M[e];
        }
        r->flags[id].store(2, std::memory_order_release);
    }
}

int check(int nbv, int nseg, int nvt, float beta, int rep) {
    Run r(nbv, nseg, nvt, beta);
    for (int bv = 0; bv < nbv; ++bv)
        for (int e = 0; e < kElems; ++e) {
            r.S0[bv].S[e] = value(-1, bv, e, 0);
            r.S0[bv].M[e] = value(-1, bv, e, 1);
        }
    std::vector<std::thread> th;
    for (int i = 0; i < nbv * nseg; ++i) th.emplace_back(workgroup, &r, i);
    for (auto& x : th) x.join();
    if (r.error.load()) {
        std::fprintf(stderr, "rep %d: a wait gave up\n", rep);
        return 1;
    }
    // reference: the same walk, single-threaded, in segment order
    std::vector<Block> agg(nbv * nseg), incl(nbv * nseg);
    for (int seg = 0; seg < nseg; ++seg)
        for (int bv = 0; bv < nbv; ++bv) {
            const int id = seg * nbv + bv;
            for (int e = 0; e < kElems; ++e) {
                agg[id].S[e] = value(seg, bv, e, 0);
                agg[id].M[e] = value(seg, bv, e, 1);
            }
            auto read = [&](int j, int bvj, int want) -> const Block& {
                return want == 2 ? incl[j * nbv + bvj] : agg[j * nbv + bvj];
            };
            const Block st = walk(r, seg, bv, read);
            for (int e = 0; e < kElems; ++e) {
                incl[id].S[e] = agg[id].S[e] + st.S[e] + r.a_seg * st.M[e];
                incl[id].M[e] = agg[id].M[e] + r.g_seg * st.M[e];
                if (st.S[e] != r.start[id].S[e] || st.M[e] != r.start[id].M[e]) {
                    std::fprintf(stderr, "rep %d: segment %d column %d entry %d differs\n", rep, seg, bv, e);
                    return 1;
                }
            }
            // the plain sequential chain (double): the state after segments < seg
            double S = 0, M = 0;
            for (int e = 0; e < kElems; ++e) {
                S = r.S0[bv].S[e];
                M = r.S0[bv].M[e];
                for (int j = 0; j < seg; ++j) {
                    S = S + r.a_seg * M + value(j, bv, e, 0);
                    M = r.g_seg * M + value(j, bv, e, 1);
                }
                const double tol = 1e-4 * (1.0 + std::fabs(S) + std::fabs(M));
                if (std::fabs(S - st.S[e]) > tol || std::fabs(M - st.M[e]) > tol) {
                    std::fprintf(stderr, "rep %d: segment %d differs from the sequential chain\n", rep, seg);
                    return 1;
                }
            }
        }
    return 0;
}

}  // namespace

int main() {
    // (nbv, nseg, tiles per head); 16 pairs of 8 heads take the grouped tickets
    const int shapes[][3] = {{2, 4, 2}, {3, 12, 1}, {1, 20, 1}, {4, 17, 2}, {16, 4, 2}, {16, 9, 2}};
    const float betas[] = {0.f, 0.9f, 0.5f};
    int fails = 0, n = 0;
    for (int rep = 0; rep < 4; ++rep)
        for (const auto& sh : shapes)
            for (float b : betas) {
                fails += check(sh[0], sh[1], sh[2], b, rep);
                ++n;
            }
    std::printf("lookback model: %d runs, %d failures\n", n, fails);
    return fails ? 1 : 0;
}
