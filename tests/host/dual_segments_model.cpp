// dual_segments_model.cpp -- a host model of the segment protocol of the
// segmented dual form, for ThreadSanitizer (CPU only, test code).
//
// Over whole mini-batches the dual form's update is affine in the state, so a
// segment maps its start state W to f_s(W) = W + (Delta_s W + B_s) ([P4] "RNN의
// 기억을 작은 모델로 바꾼다면: Test-Time Training 읽기", section on making the
// gradient an efficient layer: inside a mini-batch every gradient is taken at
// W_n).  The model keeps a few state entries per head and a diagonal Delta.
//
// Threads play workgroups.  Thread i belongs to group i % G (G = 8 when the
// heads split evenly into 8 groups, else 1) and takes a ticket from its
// group's counter; ticket t of group g runs segment t / per of head
// (t % per) G + g (per = heads / G), and marks its flag started (bit 1).
// Segment 0 runs its forward from W0 and publishes its end state (bit 0).
// Segments 1 .. n-2 publish their maps, wait for the state and the earlier
// maps, compose them onto segment 0's state and run their forward.  The last
// segment has no thread: segment 0 claims it (compare-and-swap on the last
// segment's flag) once every map producer of its head has started, composes
// maps 1 .. n-2 onto its end state and runs it; if segment 0 declines,
// segment n-2 claims it after its own forward and runs it from its end state.
// In "late" runs the threads of segment n-2 take their tickets only after
// every segment 0 has decided, which forces the second path; in "early" runs
// segment 0 decides only after every thread has taken its ticket, which
// forces the first.
// The model checks, over many runs:
//   - every segment's start state and the final state equal a
//     single-threaded sequential chain, bit for bit;
//   - exactly one thread runs each head's last segment: segment n-2's in
//     late runs, segment 0's in early runs;
//   - no wait gave up.
// Under -fsanitize=thread, any read of a map or state not ordered after its
// write by the flag's release/acquire pair is reported as a data race.
#include <atomic>
#include <cstdio>
#include <memory>
#include <thread>
#include <vector>

namespace {

constexpr int kElems = 8;
constexpr long kMaxPolls = 1L << 26;

struct Vec {
    float x[kElems];
};

float value(int head, int seg, int e, int which) {
    unsigned u = (unsigned)(head * 7919 + seg * 104729 + e * 31 + which * 1000003) * 2654435761u;
    u ^= u >> 15;
    u *= 2246822519u;
    u ^= u >> 13;
    return ((float)(u & 0xffff) / 65536.f - 0.5f) * (which ? 1.f : 0.2f);
}

// f_s(W) = W + (Delta_s W + B_s), the order the kernel's composition adds in
Vec apply(int head, int seg, const Vec& w) {
    Vec r;
    for (int e = 0; e < kElems; ++e) r.x[e] = w.x[e] + (value(head, seg, e, 0) * w.x[e] + value(head, seg, e, 1));
    return r;
}

struct Run {
    int heads, nseg, groups, per;
    int mode;   // 0 free, 1 late, 2 early
    std::vector<Vec> maps_b;                  // [heads][nseg]: a published map (its B; Delta is value())
    std::vector<Vec> state0;                  // [heads]: segment 0's end state
    std::vector<Vec> start;                   // [heads][nseg]
    std::vector<Vec> final_state;             // [heads]
    std::unique_ptr<std::atomic<int>[]> flags, tickets, last_runs, last_by;
    std::atomic<int> decided{0}, ticketed{0}, error{0};

    Run(int h, int n, int mode_) : heads(h), nseg(n), groups(h % 8 == 0 ? 8 : 1), per(h / (h % 8 == 0 ? 8 : 1)),
                                    mode(mode_) {
        maps_b.resize(h * n);
        state0.resize(h);
        start.resize(h * n);
        final_state.resize(h);
        flags.reset(new std::atomic<int>[h * n]);
        for (int i = 0; i < h * n; ++i) flags[i].store(0, std::memory_order_relaxed);
        tickets.reset(new std::atomic<int>[groups]);
        for (int g = 0; g < groups; ++g) tickets[g].store(0, std::memory_order_relaxed);
        last_runs.reset(new std::atomic<int>[h]);
        last_by.reset(new std::atomic<int>[h]);
        for (int i = 0; i < h; ++i) {
            last_runs[i].store(0, std::memory_order_relaxed);
            last_by[i].store(-1, std::memory_order_relaxed);
        }
    }
    std::atomic<int>& flag(int head, int seg) { return flags[head * nseg + seg]; }
};

Vec w0(int head) {
    Vec v;
    for (int e = 0; e < kElems; ++e) v.x[e] = value(head, -1, e, 1);
    return v;
}

void wait_published(Run* r, int head, int j_end) {
    for (int j = 0; j < j_end; ++j) {
        long polls = 0;
        while (!(r->flag(head, j).load(std::memory_order_acquire) & 1)) {
            if (++polls > kMaxPolls) {
                r->error.store(1, std::memory_order_relaxed);
                return;
            }
            std::this_thread::yield();
        }
    }
}

// the forward over the last segment from state w, by the workgroup of segment `by`
void run_last(Run* r, int head, int by, Vec w) {
    r->last_runs[head].fetch_add(1, std::memory_order_relaxed);
    r->last_by[head].store(by, std::memory_order_relaxed);
    r->start[head * r->nseg + r->nseg - 1] = w;
    r->final_state[head] = apply(head, r->nseg - 1, w);
}

bool claim(Run* r, int head) {
    int expect = 0;
    return r->flag(head, r->nseg - 1).compare_exchange_strong(expect, 1, std::memory_order_acq_rel);
}

void workgroup(Run* r, int index) {
    const int G = r->groups, grp = index % G, n = r->nseg;
    // in late runs the last `per` threads of every group, which take the
    // group's segment n-2 tickets, wait for all segment-0 decisions first
    if (r->mode == 1 && n >= 3 && index / G >= r->per * (n - 2)) {
        while (r->decided.load(std::memory_order_acquire) < r->heads) std::this_thread::yield();
    }
    const int t = r->tickets[grp].fetch_add(1, std::memory_order_relaxed);
    const int seg = t / r->per, head = (t % r->per) * G + grp;
    r->flag(head, seg).store(2, std::memory_order_relaxed);   // started
    r->ticketed.fetch_add(1, std::memory_order_relaxed);
    if (seg == 0) {
        const Vec end = apply(head, 0, w0(head));
        r->start[head * n] = w0(head);
        r->state0[head] = end;
        r->flag(head, 0).store(3, std::memory_order_release);
        if (n == 1) {
            r->final_state[head] = end;
            r->decided.fetch_add(1, std::memory_order_release);
            return;
        }
        if (r->mode == 2)
            while (r->ticketed.load(std::memory_order_relaxed) < r->heads * (n - 1)) std::this_thread::yield();
        bool ok = true;
        for (int j = 1; j < n - 1; ++j) ok = ok && (r->flag(head, j).load(std::memory_order_relaxed) & 2);
        if (ok) ok = claim(r, head);
        r->decided.fetch_add(1, std::memory_order_release);
        if (!ok) return;
        Vec w = end;
        wait_published(r, head, n - 1);
        for (int j = 1; j < n - 1; ++j) {   // compose the published maps
            const Vec& b = r->maps_b[head * n + j];
            for (int e = 0; e < kElems; ++e) w.x[e] = w.x[e] + (value(head, j, e, 0) * w.x[e] + b.x[e]);
        }
        run_last(r, head, 0, w);
        return;
    }
    // segments 1 .. n-2: publish the map, then the forward from the composed start
    r->maps_b[head * n + seg] = apply(head, seg, Vec{});        // B_s = f_s(0)
    r->flag(head, seg).store(3, std::memory_order_release);
    wait_published(r, head, seg);
    Vec w = r->state0[head];
    for (int j = 1; j < seg; ++j) {
        const Vec& b = r->maps_b[head * n + j];
        for (int e = 0; e < kElems; ++e) w.x[e] = w.x[e] + (value(head, j, e, 0) * w.x[e] + b.x[e]);
    }
    r->start[head * n + seg] = w;
    const Vec end = apply(head, seg, w);
    if (seg == n - 2) {
        // early runs: segment n-2's own forward ends after segment 0 decided,
        // as a forward that follows a map pass does in the kernel
        if (r->mode == 2)
            while (r->decided.load(std::memory_order_acquire) < r->heads) std::this_thread::yield();
        if (claim(r, head)) run_last(r, head, seg, end);
    }
}

int check(int heads, int nseg, int mode, int rep, int* fallback) {
    Run r(heads, nseg, mode);
    std::vector<std::thread> th;
    const int nwg = heads * (nseg - 1);
    for (int i = 0; i < nwg; ++i) th.emplace_back(workgroup, &r, i);
    for (auto& x : th) x.join();
    if (r.error.load()) {
        std::fprintf(stderr, "rep %d: a wait gave up\n", rep);
        return 1;
    }
    for (int h = 0; h < heads; ++h) {
        if (r.last_runs[h].load() != 1) {
            std::fprintf(stderr, "rep %d head %d: last segment ran %d times\n", rep, h, r.last_runs[h].load());
            return 1;
        }
        const int by = r.last_by[h].load();
        if (by != 0) ++*fallback;
        if (nseg > 2 && ((mode == 1 && by != nseg - 2) || (mode == 2 && by != 0))) {
            std::fprintf(stderr, "rep %d head %d: mode %d, last segment by %d\n", rep, h, mode, by);
            return 1;
        }
        Vec w = w0(h);
        for (int s = 0; s < nseg; ++s) {
            for (int e = 0; e < kElems; ++e)
                if (w.x[e] != r.start[h * nseg + s].x[e]) {
                    std::fprintf(stderr, "rep %d head %d: segment %d start differs\n", rep, h, s);
                    return 1;
                }
            w = apply(h, s, w);
        }
        for (int e = 0; e < kElems; ++e)
            if (w.x[e] != r.final_state[h].x[e]) {
                std::fprintf(stderr, "rep %d head %d: final state differs\n", rep, h);
                return 1;
            }
    }
    return 0;
}

}  // namespace

int main() {
    // (heads, segments): grouped tickets (16, 24 heads) and one counter (3, 5)
    const int shapes[][2] = {{16, 5}, {24, 3}, {3, 6}, {5, 2}, {16, 2}};
    int fails = 0, n = 0, fallback[3] = {0, 0, 0};
    for (int rep = 0; rep < 4; ++rep)
        for (const auto& sh : shapes)
            for (int mode = 0; mode < 3; ++mode) {
                fails += check(sh[0], sh[1], mode, rep, &fallback[mode]);
                ++n;
            }
    std::printf("dual segments model: %d runs, %d failures, last segment by segment n-2 in %d late, %d early "
                "and %d free heads\n", n, fails, fallback[1], fallback[2], fallback[0]);
    return fails ? 1 : 0;
}
