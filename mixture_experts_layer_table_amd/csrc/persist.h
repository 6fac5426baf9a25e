// Persistent producer/consumer scheduling of the two grouped GEMMs of a ring
// round (forward: gate/up -> down; backward: dA -> dX), in one launch of one
// workgroup per compute unit.
//
// Why ("Mixture-of-Kittens(MoK)란?" explainer, section 4 ②: overlap granularity
// is chosen per workload; "technical foundation": scheduling inside the kernel
// rather than by the host): with 256 x 256 tiles a GEMM of the EP-64 share is
// 2 to 7 waves of tiles over 256 compute units, so a stream of separate
// launches idles most of the chip during the last partial wave of every
// GEMM. Here consumer tiles of an m-tile start as soon as that m-tile's
// producer tiles are done, filling those tails.
//
// Work queue. Items of class 1 (producer tiles) and class 2 (consumer tiles)
// are numbered in the XCD-aware group order of the separate launches (groups
// of pair_group_m m-tiles x all n-tiles) and cut into 8 contiguous chunks, one per
// XCD, at whole groups: chunk x of either class covers the same m-tiles. A
// workgroup claims from its own XCD's chunk first and then from the others,
// producers before consumers. So an XCD's first consumer tiles belong to the
// m-tiles that its own first producer tiles made, done long before; a chunk
// cut inside a group would hand the next XCD, as its first consumer tiles,
// m-tiles whose last producer tiles sit at the end of this XCD's chunk
// (measured: consumer tiles then waited 17-22 us each on average).
// Claim counters are integers in the workspace, taken with atomic add.
// Completion of a producer tile is published with a release increment of its
// m-tile's counter (device scope: the write-back of this XCD's L2); a consumer
// waits until its m-tile's counter is complete, then takes an acquire fence
// (invalidate of its L2 and L1) before reading what the producers wrote.
//
// Deadlock freedom: producers depend on nothing inside the launch, and a
// consumer tile is claimed only after every producer tile has been claimed,
// i.e. is running on a resident workgroup that will finish it; a workgroup
// waiting for its consumer tile's m-tile therefore always waits for work in
// progress, whatever number of workgroups is resident. (Claiming consumers by
// fetch-and-add and then waiting, rather than polling for a ready one, keeps
// the claim itself one atomic per tile.) A poll budget bounds the wait anyway:
// exhausting it sets MOK_SCHEDULER_STALLED and exits.
//
// Results equal those of separate launches bit for bit: every output tile is
// computed by one workgroup in the same order.
#pragma once
#include "gemm8.h"
#include "layer_parts.h"

namespace mok {
namespace {

constexpr int kSpinLimit = 1 << 20;   // polls without a claim before giving up

struct PairSync {
    int *head;   // [2 * kXcds] claimed items of class 1 / 2 per XCD chunk (relative to the chunk start)
    int *done;   // [m-tiles of the round] finished producer tiles per m-tile
    int spin_limit;   // poll budget of a wait; < 0: every wait gives up at once (stall-path test)
    TraceArgs trace;  // optional per-item trace (trace.rec null: off)
};

__device__ __forceinline__ int load_relaxed(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: wait until *p >= target. Gives up (and flags the stall) after
// `limit` polls, or as soon as another workgroup has flagged one, so that a
// stalled launch ends in about one poll budget instead of one budget per
// remaining item. limit < 0 gives up at once (forced from the host to test
// this exit path).
__device__ __forceinline__ bool wait_at_least(const int *p, int target, uint32_t *status, int limit) {
    if (limit < 0) {
        atomicOr(status, MOK_SCHEDULER_STALLED);
        return false;
    }
    int polls = 0;
    while (load_relaxed(p) < target) {
        if (++polls > limit) {
            atomicOr(status, MOK_SCHEDULER_STALLED);
            return false;
        }
        if ((polls & 255) == 0 &&
            (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & MOK_SCHEDULER_STALLED))
            return false;
        __builtin_amdgcn_s_sleep(8);
    }
    return true;
}

// item id -> (m-tile j, n-tile n) in the group order of decode_seg_tile,
// with groups of gsz m-tiles
__device__ __forceinline__ void item_tile(int id, int nt, int mtc, int &j, int &n, int gsz = kGroupM) {
    const int gsize = gsz * nt, grp = id / gsize, first = grp * gsz;
    const int gm = min(gsz, mtc - first), r = id % gsize;
    j = first + r % gm;
    n = r / gm;
}

struct QueueShape {
    int mtc, nt1, nt2, n1, n2, ng;   // ng: groups of gsz m-tiles
    int gsz;                         // m-tiles per group of the item order
};

// m-tiles per group of a pair kernel's item order. Layers of many small
// experts (128-row tiles: one m-tile per expert, on average) take one, so the
// 32 compute units of an XCD share two experts' rows in its L2 instead of
// four, beside the weights streaming through it (the forward pair 2.5% faster
// on 256 experts of 64 rows); larger groups keep the segment GEMMs' order.
template <class C>
constexpr int pair_group_m() {
    return C::BM == 128 ? 1 : kGroupM;
}

// Items [start, start + len) of chunk x for a class with nt n-tiles per m-tile
// and n items: the whole groups [x*ng/8, (x+1)*ng/8).
__device__ __forceinline__ void chunk_span(const QueueShape &q, int x, int nt, int n, int &start, int &len) {
    const int g0 = x * q.ng / kXcds, g1 = (x + 1) * q.ng / kXcds;
    start = min(n, g0 * q.gsz * nt);
    len = min(n, g1 * q.gsz * nt) - start;
}

// Thread 0 of a workgroup: claim the next item. Returns its class (0: queue
// drained) and sets id. Producer tiles go first, so that the tiles an XCD runs
// together stay in the lockstep order of a separate launch (their shared
// operand slices are then read from L2, not HBM); consumer tiles fill the
// compute units that the producers' last partial wave leaves idle. A consumer
// tile is claimed only once every producer tile is claimed, i.e. running on a
// resident workgroup that will finish it; the wait for its m-tile is separate
// (wait_consumer_inputs), so that a workgroup can claim its next item while it
// still runs the current one.
__device__ int claim_item(const PairSync &s, const QueueShape &q, int xcd, int &id) {
    for (int i = 0; i < kXcds; ++i) {
        const int x = (xcd + i) % kXcds;
        int start, len;
        chunk_span(q, x, q.nt1, q.n1, start, len);
        if (load_relaxed(&s.head[x]) >= len) continue;
        const int h = atomicAdd(&s.head[x], 1);
        if (h < len) {
            id = start + h;
            return 1;
        }
    }
    for (int i = 0; i < kXcds; ++i) {
        const int x = (xcd + i) % kXcds;
        int start, len;
        chunk_span(q, x, q.nt2, q.n2, start, len);
        if (load_relaxed(&s.head[kXcds + x]) >= len) continue;
        const int h = atomicAdd(&s.head[kXcds + x], 1);
        if (h >= len) continue;
        id = start + h;
        return 2;
    }
    return 0;
}

// Thread 0, before a consumer tile starts: wait until every producer tile of
// its m-tile is done, then acquire what they wrote. False: the wait gave up
// (stall flagged).
__device__ bool wait_consumer_inputs(const PairSync &s, const QueueShape &q, int id, uint32_t *status) {
    int j, n;
    item_tile(id, q.nt2, q.mtc, j, n, q.gsz);
    if (!wait_at_least(&s.done[j], q.nt1, status, s.spin_limit)) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

// End of a work item: every wave waits for its own global stores to be
// acknowledged by the L2 before the workgroup barrier. The barrier alone waits
// for LDS traffic only, and the agent-scope release that thread 0 performs
// afterwards (L2 write-back, then the flag) covers its own wave's stores; with
// this wait it covers the whole workgroup's. The barrier also frees the LDS
// for the next item.
__device__ __forceinline__ void item_done_barrier() {
    wait_vmcnt<0>();
    __syncthreads();
}

// Returns the K loop's end time where the tile pipeline reports it (0 otherwise).
template <class P>
__device__ __forceinline__ uint64_t run_tile(P &p, uint32_t lds) {
    if constexpr (P::FP8) {
        gemm8_tile(p, lds);
        return 0;
    } else {
        return gemm_tile(p, lds);
    }
}

// One item of a pair kernel (the block-scaled pipeline for fp8 problems).
// Returns the K loop's end time.
template <class P, class F, class G>
__device__ __forceinline__ uint64_t pair_tile(P &p, uint32_t lds, F &&between, G &&publish) {
    if constexpr (P::FP8)
        return gemm8_tile(p, lds, between, publish);
    else
        return gemm_tile(p, lds, between, publish);
}

template <class P>
__device__ __forceinline__ SegTile seg_tile(const SchedView &v, int lo, int j, int n, int64_t n_slots) {
    SegTile t;
    t.mt = v.mtiles[lo + j];
    t.nt = n;
    t.slot = (int)(t.mt.g % n_slots);
    t.rowoff = t.mt.q0 - v.mb_start[t.mt.g];
    return t;
}

// P1 tiles of m-tile j write what P2 tiles of m-tile j read (all of P1's
// n-tiles). TILE_LDS: LDS bytes of the larger tile pipeline; two ints after it
// broadcast the claimed item.
template <class P1, class P2, size_t TILE_LDS>
__global__ __launch_bounds__(P1::C::NT) void persist_pair_kernel(typename P1::Args a1, typename P2::Args a2,
                                                                 PairSync s) {
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_raw;
    int *bcast = reinterpret_cast<int *>(lds_raw + TILE_LDS);
    const SchedView &v = a1.v;
    if (*v.status) return;
    const int lo = v.mtfirst[a1.g0];
    QueueShape q;
    q.mtc = v.mtfirst[a1.g1] - lo;
    q.nt1 = a1.n_tiles;
    q.nt2 = a2.n_tiles;
    q.n1 = q.mtc * q.nt1;
    q.n2 = q.mtc * q.nt2;
    q.gsz = pair_group_m<typename P1::C>();
    q.ng = (q.mtc + q.gsz - 1) / q.gsz;
    const int xcd = (int)(blockIdx.x % kXcds);   // workgroups are dispatched round-robin over the XCDs
    uint64_t t_claim = 0, t_start = 0;   // thread 0's item-trace times
    // Thread 0 takes a ticket from its own XCD's chunk (producer chunk until
    // claim_item has once handed it a consumer tile, consumer chunk after
    // that) while the current item is in its epilogue: the atomic's round
    // trip then overlaps the epilogue instead of following it. The ticket is
    // checked at the top of the next iteration; an exhausted chunk falls back
    // to claim_item's full search, which keeps the producers-first order
    // (a consumer ticket is only ever taken once every producer tile has been
    // claimed). The wait for a consumer tile's inputs comes after the current
    // item is published: the current item may be one of the producer tiles it
    // waits for.
    int ticket = -1;   // thread 0: own-chunk ticket taken during the last epilogue (-1: none)
    int phase = 1;     // thread 0: class of the chunk the ticket came from
    for (;;) {
        if (threadIdx.x == 0) {
            if (s.trace.rec && ticket < 0) t_claim = __builtin_amdgcn_s_memrealtime();
            int cls = 0, id = 0;
            if (ticket >= 0) {
                int start, len;
                if (phase == 1) chunk_span(q, xcd, q.nt1, q.n1, start, len);
                else chunk_span(q, xcd, q.nt2, q.n2, start, len);
                if (ticket < len) {
                    cls = phase;
                    id = start + ticket;
                }
            }
            if (cls == 0) cls = claim_item(s, q, xcd, id);
            if (cls != 0) phase = cls;
            if (cls == 2 && !wait_consumer_inputs(s, q, id, v.status)) cls = 0;
            bcast[0] = cls;
            bcast[1] = id;
            if (s.trace.rec) t_start = __builtin_amdgcn_s_memrealtime();
        }
        __syncthreads();
        const int cls = bcast[0], id = bcast[1];
        if (cls == 0) return;
        uint64_t t_next = 0;
        auto take_ticket = [&]() {
            if (threadIdx.x == 0) {
                if (s.trace.rec) t_next = __builtin_amdgcn_s_memrealtime();
                ticket = atomicAdd(&s.head[(phase == 1 ? 0 : kXcds) + xcd], 1);
            }
        };
        int j, n;
        uint64_t t_kloop;
        if (cls == 1) {
            item_tile(id, q.nt1, q.mtc, j, n, q.gsz);
            P1 p;
            p.init(a1, seg_tile<P1>(v, lo, j, n, a1.n_slots));
            // the release covers every wave's stores issued before it: a split
            // epilogue issues what consumer tiles read first, the rest after
            t_kloop = pair_tile(p, lds, take_ticket, [&] {
                item_done_barrier();
                if (threadIdx.x == 0)
                    __hip_atomic_fetch_add(&s.done[j], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            });
        } else {
            item_tile(id, q.nt2, q.mtc, j, n, q.gsz);
            P2 p;
            p.init(a2, seg_tile<P2>(v, lo, j, n, a2.n_slots));
            t_kloop = pair_tile(p, lds, take_ticket, [] {});
        }
        if (cls == 2 || split_epilogue<P1>::value) {
            // Stores that nothing in this launch reads (a consumer tile's
            // output, a split producer's second part) drain while the next item
            // starts. The barrier only frees the LDS (every wave's own LDS
            // accesses done first); stores still in flight make the next
            // item's load-counter waits stricter, never weaker.
            wait_lgkm0();
            lds_barrier();
        }
        if (threadIdx.x == 0) {
            trace_item(s.trace, t_claim, t_start, t_kloop, cls, id);
            t_claim = t_next;
        }
    }
}

// ----------------------------------------------------------------------------- whole pass (k == 1)

// One launch for a whole pass when every token has one routed row: the ring
// rounds run back to back through the ring protocol instead of stream order
// ("Mixture-of-Kittens(MoK)란?" explainer, section 4 ③: a fixed ring of
// mini-batch slots, reused without the host).
//
// Items, in one global order (round r = 0 .. NR-1, rounds of S mini-batches
// ascending in the forward pass and descending in the backward pass):
//   segment 3r     gather items: 64 rows of one mini-batch g into slot g % n_slots
//   segment 3r + 1 producer tiles of the round's m-tiles (gate/up, or dA)
//   segment 3r + 2 consumer tiles of the round's m-tiles (down, or dX)
// Ring protocol, integers in the workspace:
//   full[r]      gather items of round r done  (producer tiles of round r wait
//                for all of them, so that a workgroup takes one acquire fence
//                per round instead of one per tile: each fence empties its
//                XCD's L2, which the tiles running there share)
//   done[m]      producer tiles of m-tile m done (its consumer tiles wait for all)
//   used[g]      slot-reading tiles of g done  (the last one releases the slot)
//   released[s]  mini-batches that have left slot s; a gather item of round r
//                waits until released[s] >= r (each earlier round held one
//                mini-batch in every slot)
// The slot-reading tiles are the consumers in the forward pass (down reads the
// a-ring) and the producers in the backward pass (dA reads the dy ring).
//
// A workgroup claims from segment s only after it has seen every item of the
// segments before s claimed; every item depends only on items of earlier
// segments, which are therefore running on resident workgroups or done, so
// every wait ends (by induction over the order), whatever number of
// workgroups is resident.
struct PassSync {
    int *head;       // [3 * NR * kXcds] claimed items per segment and XCD chunk
    int *full;       // [NR]
    int *used;       // [G]
    int *released;   // [min(n_slots, G)]
    int *done;       // [m-tiles]
    int spin_limit;  // as in PairSync
};

struct PassShape {
    int G, S, NR, cpm;   // mini-batches, per round, rounds, gather items per mini-batch
    bool reverse;
};

constexpr int kGatherRows = 64;   // rows per gather item (8 waves x 8 rows)

__device__ __forceinline__ void round_span(const PassShape &ps, int r, int &a, int &b) {
    if (!ps.reverse) {
        a = r * ps.S;
        b = min(ps.G, a + ps.S);
    } else {
        b = ps.G - r * ps.S;
        a = max(0, b - ps.S);
    }
}

struct PassItem {
    int kind;   // 0 none, 1 gather, 2 producer, 3 consumer
    int a, b;   // (gather) mini-batch, row chunk; (tiles) m-tile (global index), n-tile
    int round;
    int acquire;   // the item's inputs were published by other workgroups since this one last acquired
};


// Thread 0: claim the next item at or after segment `seg` and wait for its inputs.
__device__ PassItem claim_pass_item(const PassSync &s, const PassShape &ps, const SchedView &v, int nt1, int nt2,
                                    int64_t n_slots, int xcd, int &seg, int &acq_round) {
    PassItem it{0, 0, 0, 0, 0};
    for (; seg < 3 * ps.NR; ++seg) {
        const int r = seg / 3, c = seg % 3;
        int a, b;
        round_span(ps, r, a, b);
        int *head = s.head + seg * kXcds;
        if (c == 0) {
            const int n = (b - a) * ps.cpm;
            if (load_relaxed(head) >= n) continue;
            const int h = atomicAdd(head, 1);
            if (h >= n) continue;
            const int g = a + h / ps.cpm;
            if (!wait_at_least(&s.released[g % n_slots], r, v.status, s.spin_limit)) return it;
            it = PassItem{1, g, h % ps.cpm, r, 0};
            return it;
        }
        const int lo = v.mtfirst[a], mtc = v.mtfirst[b] - lo, nt = c == 1 ? nt1 : nt2;
        const int n = mtc * nt, per = (n + kXcds - 1) / kXcds;
        for (int i = 0; i < kXcds; ++i) {
            const int x = (xcd + i) % kXcds, start = x * per, len = min(n - start, per);
            if (load_relaxed(&head[x]) >= len) continue;
            const int h = atomicAdd(&head[x], 1);
            if (h >= len) continue;
            int j, nn;
            item_tile(start + h, nt, mtc, j, nn);
            int acquire = 1;
            if (c == 1) {
                if (acq_round < r) {   // first producer tile of this round on this workgroup
                    if (!wait_at_least(&s.full[r], (b - a) * ps.cpm, v.status, s.spin_limit)) return it;
                    acq_round = r;
                } else {
                    acquire = 0;
                }
            } else {
                if (!wait_at_least(&s.done[lo + j], nt1, v.status, s.spin_limit)) return it;
            }
            it = PassItem{c == 1 ? 2 : 3, lo + j, nn, r, acquire};
            return it;
        }
    }
    return it;
}

// GA: the dispatch copy (row(g, r) by one wave); P1 -> P2 as in persist_pair_kernel;
// RELEASE: the class (2 producer, 3 consumer) whose tiles are the last readers of a slot.
template <class GA, class P1, class P2, int RELEASE, size_t TILE_LDS>
__global__ __launch_bounds__(P1::C::NT) void persist_pass_kernel(GA ga, typename P1::Args a1, typename P2::Args a2,
                                                                 PassSync s, PassShape ps) {
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_raw;
    int *bcast = reinterpret_cast<int *>(lds_raw + TILE_LDS);
    const SchedView &v = a1.v;
    if (*v.status) return;
    const int xcd = (int)(blockIdx.x % kXcds);
    const int64_t n_slots = a1.n_slots;
    int seg = 0;          // thread 0's claim cursor
    int acq_round = -1;   // last round whose gathers thread 0 has acquired
    for (;;) {
        if (threadIdx.x == 0) {
            const PassItem it = claim_pass_item(s, ps, v, a1.n_tiles, a2.n_tiles, n_slots, xcd, seg, acq_round);
            bcast[0] = it.kind;
            bcast[1] = it.a;
            bcast[2] = it.b;
            bcast[3] = it.round;
            bcast[4] = it.acquire;
        }
        __syncthreads();
        const int kind = bcast[0], ia = bcast[1], ib = bcast[2];
        if (kind == 0) return;
        // Every wave takes the acquire itself, so that its own loads are
        // ordered after its own L1/L2 invalidate. Ring slots are reused within
        // this launch: this XCD's L2 and this CU's L1 may hold a slot's lines
        // from an earlier round.
        if (bcast[4]) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (kind == 1) {
            const int r0 = ib * kGatherRows;
            const int nrows = max(0, min(kGatherRows, v.mb_start[ia + 1] - v.mb_start[ia] - r0));
            int *tok = bcast + 16;   // kGatherRows token indices
            if ((int)threadIdx.x < nrows) tok[threadIdx.x] = v.perm[v.mb_start[ia] + r0 + threadIdx.x] / ga.k;
            __syncthreads();
            ga.template rows<P1::C::NT>(ia, r0, nrows, tok);
        } else if (kind == 2) {
            P1 p;
            const MTile mt = v.mtiles[ia];
            p.init(a1, SegTile{mt, ib, (int)(mt.g % n_slots), mt.q0 - v.mb_start[mt.g]});
            run_tile(p, lds);
        } else {
            P2 p;
            const MTile mt = v.mtiles[ia];
            p.init(a2, SegTile{mt, ib, (int)(mt.g % n_slots), mt.q0 - v.mb_start[mt.g]});
            run_tile(p, lds);
        }
        // Every wave writes its own stores back to where other XCDs read them
        // before the workgroup publishes the item.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        item_done_barrier();
        if (threadIdx.x == 0) {
            if (kind == 1) {
                __hip_atomic_fetch_add(&s.full[bcast[3]], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                if (kind == 2) __hip_atomic_fetch_add(&s.done[ia], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                if (kind == RELEASE) {
                    const int g = v.mtiles[ia].g;
                    const int expect = (v.mtfirst[g + 1] - v.mtfirst[g]) * (kind == 2 ? a1.n_tiles : a2.n_tiles);
                    const int prev = __hip_atomic_fetch_add(&s.used[g], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                    if (prev + 1 == expect)
                        __hip_atomic_fetch_add(&s.released[g % n_slots], 1, __ATOMIC_RELEASE,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
}

// Clears the claim and completion counters (a kernel, so that a captured
// graph replays it).
__global__ __launch_bounds__(256) void sync_clear(int *p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

inline int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    return n;
}

// Workgroups of a persistent launch: the plan's cap, else one per compute unit.
inline unsigned persistent_grid(const Plan &p) { return (unsigned)(p.grid > 0 ? p.grid : device_cu_count()); }

// Sync-area layout of the whole-pass kernel, in ints.
struct PassLayout {
    int NR, S, cpm, slots, total;
    int head, full, used, released, done;
};
inline PassLayout pass_layout(const Plan &p) {
    PassLayout l;
    l.S = (int)std::min<int64_t>(p.n_slots, (int64_t)p.G);
    l.NR = p.G == 0 ? 0 : (p.G + l.S - 1) / l.S;
    l.cpm = (p.MB + kGatherRows - 1) / kGatherRows;
    l.slots = l.S;
    l.head = 0;
    l.full = l.head + 3 * l.NR * kXcds;
    l.used = l.full + l.NR;
    l.released = l.used + p.G;
    l.done = l.released + l.slots;
    l.total = l.done + (int)p.max_mtiles;
    return l;
}

// Poll budget of the persistent kernels' waits (MOK_DEBUG_FORCE_STALL: none).
inline int spin_limit(const Plan &p) { return (p.debug & MOK_DEBUG_FORCE_STALL) ? -1 : kSpinLimit; }

template <class GA, class P1, class P2, int RELEASE, size_t TILE_LDS>
hipError_t launch_pass(const char *name, const Plan &p, const GA &ga, const typename P1::Args &a1,
                       const typename P2::Args &a2, bool reverse, int *sync, hipStream_t st) {
    constexpr size_t lds_bytes = TILE_LDS + 64 + 4 * kGatherRows;   // claim broadcast, gather token ids
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)persist_pass_kernel<GA, P1, P2, RELEASE, TILE_LDS>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const PassLayout l = pass_layout(p);
    sync_clear<<<(unsigned)std::min<int64_t>((l.total + 255) / 256, 1024), 256, 0, st>>>(sync, l.total);
    const PassSync s{sync + l.head, sync + l.full, sync + l.used, sync + l.released, sync + l.done, spin_limit(p)};
    const PassShape ps{p.G, l.S, l.NR, l.cpm, reverse};
    KernelTimer tm(name, st);
    persist_pass_kernel<GA, P1, P2, RELEASE, TILE_LDS>
        <<<persistent_grid(p), P1::C::NT, lds_bytes, st>>>(ga, a1, a2, s, ps);
    return hipGetLastError();
}

template <class P1, class P2, size_t TILE_LDS>
hipError_t launch_pair(const char *name, const typename P1::Args &a1, const typename P2::Args &a2, int *sync,
                       int64_t max_mtiles, int spin, unsigned grid, hipStream_t st, TraceArgs tr) {
    constexpr size_t lds_bytes = TILE_LDS + 64;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)persist_pair_kernel<P1, P2, TILE_LDS>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int n = kSyncHeads + (int)max_mtiles;
    sync_clear<<<(unsigned)std::min<int64_t>((n + 255) / 256, 1024), 256, 0, st>>>(sync, n);
    KernelTimer tm(name, st);
    persist_pair_kernel<P1, P2, TILE_LDS>
        <<<grid, P1::C::NT, lds_bytes, st>>>(a1, a2, PairSync{sync, sync + kSyncHeads, spin, tr});
    return hipGetLastError();
}

}  // namespace
}  // namespace mok
