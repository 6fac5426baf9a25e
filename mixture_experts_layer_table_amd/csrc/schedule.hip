// Device-side schedule builder: one table drives every phase of both passes
// ("Mixture-of-Kittens(MoK)란?" explainer, section 4 ①), built without any
// device-to-host read and without dropping a routed row (section 4 ③).
//
// Processing order sorts routed rows f = t*k + j by (macro-batch, expert, f).
// With rank_e(f) = #{f' < f : id(f') = e} (a stable counting sort), the
// position of f in macro-batch m is
//     q(f) = moffsets[m][e] + rank_e(f) - rank_e(first row of m),
// and its position in canonical (expert, f) order is offsets[e] + rank_e(f).
// Only integer atomics are used (order-independent counts).
#include "kernels.h"
#include "timing.h"
#include "views.h"

namespace mok {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void sched_init(SchedView v) {
    if (threadIdx.x == 0) {
        *v.status = 0;
        *v.n_seg = 0;
        *v.fprint = v.fingerprint;
    }
    // defined values for an empty call (T = 0), where the scan does not run
    for (int e = threadIdx.x; e <= v.E; e += kThreads) {
        if (e < v.E) v.counts[e] = 0;
        v.offsets[e] = 0;
    }
}

// Per-chunk expert histogram; flags ids outside [0, E).
__global__ __launch_bounds__(kThreads) void sched_hist(const int32_t *__restrict__ ids, SchedView v) {
    extern __shared__ int hist[];
    for (int e = threadIdx.x; e < v.E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kSchedChunk;
    bool bad = false;
    for (int r = threadIdx.x; r < kSchedChunk; r += kThreads) {
        const int f = base + r;
        if (f < v.R) {
            const int id = ids[f];
            if ((unsigned)id >= (unsigned)v.E)
                bad = true;
            else
                atomicAdd(&hist[id], 1);
        }
    }
    if (bad) atomicOr(v.status, MOK_BAD_EXPERT_ID);
    __syncthreads();
    for (int e = threadIdx.x; e < v.E; e += kThreads) v.chunk[blockIdx.x * v.E + e] = hist[e];
}

constexpr int kTableThreads = 1024;

// Exclusive scan of a[0, n) in place by one block of kTableThreads threads
// (each thread a contiguous run, then a scan of the run totals); returns the
// total. Every thread of the block must call it.
__device__ int block_exclusive_scan1(int *a, int n) {
    __shared__ int s[kTableThreads];
    const int tid = threadIdx.x;
    const int per = (n + kTableThreads - 1) / kTableThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int x = 0;
    for (int i = lo; i < hi; ++i) x += a[i];
    s[tid] = x;
    __syncthreads();
    for (int d = 1; d < kTableThreads; d <<= 1) {
        const int y = tid >= d ? s[tid - d] : 0;
        __syncthreads();
        s[tid] += y;
        __syncthreads();
    }
    int r = tid ? s[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        const int t = a[i];
        a[i] = r;
        r += t;
    }
    const int tot = s[kTableThreads - 1];
    __syncthreads();
    return tot;
}

// Exclusive scan of each expert's chunk histogram over chunks; counts, offsets.
// The chunk counts are loaded a batch at a time and the offsets come from a
// block scan: with hundreds of experts, one thread walking them (or a chunk
// list one dependent load at a time) was most of the schedule's time.
__global__ __launch_bounds__(kTableThreads) void sched_scan(SchedView v) {
    if (*v.status) return;
    constexpr int B = 8;
    for (int e = threadIdx.x; e < v.E; e += kTableThreads) {
        int run = 0;
        for (int c0 = 0; c0 < v.nchunks; c0 += B) {
            int t[B];
#pragma unroll
            for (int i = 0; i < B; ++i) t[i] = c0 + i < v.nchunks ? v.chunk[(c0 + i) * v.E + e] : 0;
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (c0 + i < v.nchunks) {
                    v.chunk[(c0 + i) * v.E + e] = run;
                    run += t[i];
                }
        }
        v.counts[e] = run;
        v.offsets[e] = run;
    }
    __syncthreads();
    const int tot = block_exclusive_scan1(v.offsets, v.E);
    if (threadIdx.x == 0) v.offsets[v.E] = tot;
}

// rank_e at the first routed row of each macro-batch (and at R).
__global__ __launch_bounds__(kThreads) void sched_bounds(const int32_t *__restrict__ ids, SchedView v) {
    if (*v.status) return;
    extern __shared__ int hist[];
    const int b = blockIdx.x;
    const int64_t fb64 = (int64_t)b * v.k * v.MT;
    const int fb = (int)(fb64 < v.R ? fb64 : v.R);
    const int c = fb / kSchedChunk;
    for (int e = threadIdx.x; e < v.E; e += kThreads) hist[e] = 0;
    __syncthreads();
    for (int r = c * kSchedChunk + threadIdx.x; r < fb; r += kThreads) atomicAdd(&hist[ids[r]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < v.E; e += kThreads)
        v.bound[b * v.E + e] = (c < v.nchunks ? v.chunk[c * v.E + e] : v.counts[e]) + hist[e];
}

struct MbRange {
    int m, q_lo, q_hi;
};

__device__ MbRange minibatch_range(const SchedView &v, int g) {
    const int m = g / v.nb_full, b = g % v.nb_full;
    const int t0 = m * v.MT;
    const int t1 = min(v.T, t0 + v.MT);
    const int base = v.k * t0, rm = v.k * (t1 - t0);
    return MbRange{m, base + b * v.MB, base + min(rm, (b + 1) * v.MB)};
}

// Largest e in [0, E) with M[e] <= q (M non-decreasing, M[0] <= q).
__device__ int expert_at(const int32_t *M, int E, int q) {
    int lo = 0, hi = E;   // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (M[mid] <= q) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ void block_exclusive_scan2(int *a, int *b, int G, int &tot_a, int &tot_b) {
    __shared__ int sa[kTableThreads], sb[kTableThreads];
    const int tid = threadIdx.x;
    const int per = (G + kTableThreads - 1) / kTableThreads;
    const int lo = min(G, tid * per), hi = min(G, lo + per);
    int xa = 0, xb = 0;
    for (int i = lo; i < hi; ++i) {
        xa += a[i];
        xb += b[i];
    }
    sa[tid] = xa;
    sb[tid] = xb;
    __syncthreads();
    for (int d = 1; d < kTableThreads; d <<= 1) {
        const int ya = tid >= d ? sa[tid - d] : 0, yb = tid >= d ? sb[tid - d] : 0;
        __syncthreads();
        sa[tid] += ya;
        sb[tid] += yb;
        __syncthreads();
    }
    int ra = tid ? sa[tid - 1] : 0, rb = tid ? sb[tid - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        const int ta = a[i], tb = b[i];
        a[i] = ra;
        b[i] = rb;
        ra += ta;
        rb += tb;
    }
    tot_a = sa[kTableThreads - 1];
    tot_b = sb[kTableThreads - 1];
    __syncthreads();
}

// Macro-batch offsets, mini-batch ranges, segments and m-tiles (one block).
__global__ __launch_bounds__(kTableThreads) void sched_table(SchedView v) {
    if (*v.status) return;
    const int tid = threadIdx.x;
    if (v.E > 64 && v.NM <= 64) {   // many experts, few macro-batches: a block scan per macro-batch
        for (int m = 0; m < v.NM; ++m) {
            int32_t *M = v.moffsets + m * (v.E + 1);
            for (int e = tid; e < v.E; e += kTableThreads) {
                const int mc = v.bound[(m + 1) * v.E + e] - v.bound[m * v.E + e];
                v.mcounts[m * v.E + e] = mc;
                M[e] = mc;
            }
            __syncthreads();
            const int base = m * v.MT * v.k, tot = block_exclusive_scan1(M, v.E);
            for (int e = tid; e < v.E; e += kTableThreads) M[e] += base;
            if (tid == 0) M[v.E] = base + tot;
        }
    } else {   // one thread per macro-batch walks its experts
        for (int m = tid; m < v.NM; m += kTableThreads) {
            int run = m * v.MT * v.k;
            for (int e = 0; e < v.E; ++e) {
                const int mc = v.bound[(m + 1) * v.E + e] - v.bound[m * v.E + e];
                v.mcounts[m * v.E + e] = mc;
                v.moffsets[m * (v.E + 1) + e] = run;
                run += mc;
            }
            v.moffsets[m * (v.E + 1) + v.E] = run;
        }
    }
    __syncthreads();
    for (int g = tid; g < v.G; g += kTableThreads) {
        const MbRange r = minibatch_range(v, g);
        const int32_t *M = v.moffsets + r.m * (v.E + 1);
        int ns = 0, nt = 0;
        for (int e = expert_at(M, v.E, r.q_lo); e < v.E && M[e] < r.q_hi; ++e) {
            const int len = min(r.q_hi, M[e + 1]) - max(r.q_lo, M[e]);
            if (len > 0) {
                ++ns;
                nt += (len + v.BM - 1) / v.BM;
            }
        }
        v.segfirst[g] = ns;
        v.mtfirst[g] = nt;
    }
    __syncthreads();
    int n_seg = 0, n_mt = 0;
    block_exclusive_scan2(v.segfirst, v.mtfirst, v.G, n_seg, n_mt);
    const bool overflow = n_seg > v.cap;
    if (tid == 0) {
        *v.n_seg = n_seg;
        if (overflow) atomicOr(v.status, MOK_SCHEDULE_OVERFLOW);
        v.segfirst[v.G] = n_seg;
        v.mtfirst[v.G] = n_mt;
        v.mb_start[v.G] = v.R;
    }
    for (int g = tid; g < v.G; g += kTableThreads) {
        const MbRange r = minibatch_range(v, g);
        v.mb_start[g] = r.q_lo;
        const int32_t *M = v.moffsets + r.m * (v.E + 1);
        int s = v.segfirst[g], t = v.mtfirst[g];
        for (int e = expert_at(M, v.E, r.q_lo); e < v.E && M[e] < r.q_hi; ++e) {
            const int a = max(r.q_lo, M[e]);
            const int len = min(r.q_hi, M[e + 1]) - a;
            if (len <= 0) continue;
            if (s < v.cap) {
                int4 sg = make_int4(g, e, a, len);
                reinterpret_cast<int4 *>(v.segments)[s] = sg;
            }
            ++s;
            if (!overflow) {
                // canonical position of q = a: rows of e in earlier macro-batches come first
                const int c_a = v.offsets[e] + v.bound[r.m * v.E + e] + (a - M[e]);
                for (int j = 0; j * v.BM < len; ++j, ++t) {
                    if (t < v.max_mtiles)
                        v.mtiles[t] = MTile{a + j * v.BM, min(v.BM, len - j * v.BM), e, g, c_a + j * v.BM, 0, 0, 0};
                }
            }
        }
    }
}

// Stable scatter: perm, inv, canon, ctok. A block ranks its chunk's rows in
// row order, 256 rows (one per thread) at a time: inside a wave, the lanes
// holding one expert are grouped with ballots (one pass per distinct expert
// of the wave), which gives each row its rank among the wave's rows of its
// expert and the group's size; the waves then take their turn, in order, at
// a shared per-expert count of the rows already ranked in this chunk. With
// the chunk's start count per expert (sched_bounds) that is the row's stable
// rank among all rows of its expert.
__global__ __launch_bounds__(kThreads) void sched_scatter(const int32_t *__restrict__ ids, SchedView v) {
    if (*v.status) return;
    extern __shared__ int s_cnt[];   // [E] rows of each expert ranked so far in this chunk
    const int base = blockIdx.x * kSchedChunk;
    const int n = min(kSchedChunk, v.R - base);
    for (int e = threadIdx.x; e < v.E; e += kThreads) s_cnt[e] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;   // lanes below this one
    for (int r0 = 0; r0 < n; r0 += kThreads) {
        const int r = r0 + (int)threadIdx.x;
        const bool live = r < n;
        const int e = live ? ids[base + r] : -1;
        // group the wave's lanes by expert: each pass takes the lowest remaining lane's expert
        uint64_t rest = __ballot(live);
        int rank_w = 0, leader = 0, count = 0;
        while (rest) {
            const int l0 = __ffsll((unsigned long long)rest) - 1;
            const int e0 = __shfl(e, l0);
            const uint64_t grp = __ballot(live && e == e0) & rest;
            if (live && e == e0) {
                rank_w = __popcll(grp & lt);
                leader = l0;
                count = __popcll(grp);
            }
            rest &= ~grp;
        }
        // the waves of this step take their turn at the shared counts in row order
        int start = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            __syncthreads();
            if (wave == w && live && lane == leader) {
                start = s_cnt[e];
                s_cnt[e] = start + count;
            }
        }
        start = __shfl(start, leader);
        if (live) {
            const int rank = v.chunk[blockIdx.x * v.E + e] + start + rank_w;
            const int f = base + r;
            const int t = f / v.k;
            const int m = t / v.MT;
            const int q = v.moffsets[m * (v.E + 1) + e] + rank - v.bound[m * v.E + e];
            const int c = v.offsets[e] + rank;
            if ((unsigned)q < (unsigned)v.R && (unsigned)c < (unsigned)v.R) {   // always (the ranks are a permutation)
                v.perm[q] = f;
                v.inv[f] = q;
                v.canon[c] = q;
                v.ctok[c] = t;
            }
        }
        __syncthreads();   // this step's counts are complete before the next step reads them
    }
}

// A reader's check of the table before anything else reads it: a table whose
// fingerprint differs from the reader's plan (built under other knobs or
// another shape) raises MOK_SCHEDULE_MISMATCH, and every later kernel of the
// call exits on the status word.
__global__ __launch_bounds__(64) void sched_check(uint32_t *status, const uint32_t *fprint, uint32_t expect) {
    if (threadIdx.x == 0 && *fprint != expect) atomicOr(status, MOK_SCHEDULE_MISMATCH);
}

}  // namespace

mok_status launch_schedule_check(const Plan &p, const void *schedule, hipStream_t st) {
    char *b = static_cast<char *>(const_cast<void *>(schedule));
    KernelTimer tm("sched_check", st);
    sched_check<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t *>(b + p.s_status),
                                  reinterpret_cast<const uint32_t *>(b + p.s_fprint), p.fingerprint);
    return check_hip(hipGetLastError(), "schedule check");
}

mok_status launch_build_schedule(const Plan &p, const int32_t *ids, void *schedule, hipStream_t st) {
    SchedView v = make_sched_view(p, schedule);
    const size_t hist_lds = sizeof(int) * (size_t)p.E;
    KernelTimer tm("schedule", st);
    sched_init<<<1, kThreads, 0, st>>>(v);
    if (p.nchunks > 0) {
        sched_hist<<<p.nchunks, kThreads, hist_lds, st>>>(ids, v);
        sched_scan<<<1, kTableThreads, 0, st>>>(v);
        sched_bounds<<<p.NM + 1, kThreads, hist_lds, st>>>(ids, v);
    }
    sched_table<<<1, kTableThreads, 0, st>>>(v);
    if (p.nchunks > 0) sched_scatter<<<p.nchunks, kThreads, (size_t)p.E * sizeof(int), st>>>(ids, v);
    return check_hip(hipGetLastError(), "mok_build_schedule");
}

}  // namespace mok
