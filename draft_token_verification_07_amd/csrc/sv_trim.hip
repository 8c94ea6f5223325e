// sv_trim.hip -- the vocabulary-trim d2t builder.
//
// The 2.16x EAGLE blog, sec. 6: from the token frequencies of a corpus, keep
// the core vocabulary whose cumulative probability reaches P >= 0.95, so the
// draft head scores only those ids (the SSD guide, sec. 6, scatters them back
// into the target vocabulary through d2t).  Ids in [0, Vt) are counted,
// ordered by count descending with lower ids first, and the smallest prefix
// whose count sum reaches P * (valid tokens) is kept; ids of count 0 never
// are.  d2t lists the kept ids in ascending order (the map verification
// takes) and t2d is its inverse.
//
// Three launches:
//   trim_part_kernel: workgroup (r, s) counts the ids of range r (kTrimBins
//     ids, an LDS histogram) in slice s of the stream and stores the partial
//     histogram, coalesced.  The workgroups of one slice run on one XCD (the
//     block order puts them kTrimSlices apart), so the slice is read from HBM
//     once and from that XCD's L2 by the other ranges.  No global atomics.
//   trim_reduce_kernel: sums the partial histograms of every id.
//   trim_select_kernel: one workgroup selects the cut exactly in integers: a
//     radix select over the 32-bit counts (8-bit digits, count and mass
//     histograms in LDS, each wave adding its most common digit at once)
//     finds the count c* at which the mass from the top reaches P * N and how
//     many ids of count c* are needed, the lowest ids on c* are taken, and a
//     scan over the ids writes d2t and t2d.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

constexpr int kTrimPartThreads = 512;
constexpr int kTrimPartUnroll = 8;        // 16-byte vectors in flight per thread
constexpr int kTrimSelThreads = 512;
constexpr int kTrimSelUnroll = 8;         // counts in flight per thread
constexpr int kTrimDigitBits = 11;        // radix digits: 11 + 11 + 10 bits
constexpr int kTrimDigits = 1 << kTrimDigitBits;

// Workgroup (r, s): the ids of range r in slice s of the stream.  The stream
// is read as 16-byte vectors (4 ids), kTrimPartUnroll per thread in flight;
// the ids before the first 16-byte boundary go to slice 0, those after the
// last full vector to the last slice.
template <int NT, int U>
__global__ __launch_bounds__(NT) void trim_part_kernel(TrimArgs a) {
    __shared__ uint32_t s_h[kTrimBins];
    __shared__ uint32_t s_inv;
    const int32_t r = blockIdx.x / a.S, sl = blockIdx.x % a.S;
    const int32_t id0 = r * kTrimBins;
    const int32_t nb = min(kTrimBins, a.Vt - id0);
    for (int k = threadIdx.x; k < kTrimBins; k += NT) s_h[k] = 0;
    if (threadIdx.x == 0) s_inv = 0;
    __syncthreads();
    uint32_t invalid = 0;
    auto one = [&](int32_t t) {
        const int32_t k = t - id0;
        if ((uint32_t)k < (uint32_t)nb) atomicAdd(&s_h[k], 1u);
        else if (r == 0 && (t < 0 || t >= a.Vt)) ++invalid;          // counted once, by range 0
    };
    const uintptr_t base = reinterpret_cast<uintptr_t>(a.tokens);
    int64_t head = (int64_t)(((16u - (uint32_t)(base & 15u)) & 15u) / 4u);
    if (head > a.N) head = a.N;
    const int64_t nvec = (a.N - head) / 4;
    const int64_t tail0 = head + nvec * 4;
    if (sl == 0 && (int64_t)threadIdx.x < head) one(a.tokens[threadIdx.x]);
    if (sl == a.S - 1 && (int64_t)threadIdx.x < a.N - tail0) one(a.tokens[tail0 + threadIdx.x]);
    const u32x4 *body = reinterpret_cast<const u32x4 *>(a.tokens + head);
    const int64_t v0 = nvec * sl / a.S, v1 = nvec * (sl + 1) / a.S;
    for (int64_t v = v0 + threadIdx.x; v < v1; v += (int64_t)U * NT) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = v + (int64_t)u * NT;
            raw[u] = __builtin_nontemporal_load(&body[j < v1 ? j : v1 - 1]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v + (int64_t)u * NT < v1) {
                one((int32_t)raw[u].x);
                one((int32_t)raw[u].y);
                one((int32_t)raw[u].z);
                one((int32_t)raw[u].w);
            }
    }
    if (r == 0 && invalid) atomicAdd(&s_inv, invalid);
    __syncthreads();
    uint32_t *dst = a.part + (size_t)sl * a.Vt + id0;
    for (int k = threadIdx.x; k < nb; k += NT) dst[k] = s_h[k];
    if (r == 0 && threadIdx.x == 0 && s_inv) atomicAdd(&a.totals[1], (unsigned long long)s_inv);
}

// counts[t] = sum over the slices of the partial counts of t (eight loads in
// flight per thread); the total goes to totals[0] (one atomic per workgroup)
template <int NT>
__global__ __launch_bounds__(NT) void trim_reduce_kernel(TrimArgs a) {
    constexpr int NW = NT / kWave;
    __shared__ uint64_t s_w[NW];
    const int32_t t = blockIdx.x * NT + threadIdx.x;
    uint32_t c = 0;
    if (t < a.Vt) {
        int32_t sl = 0;
        for (; sl + 8 <= a.S; sl += 8) {
            uint32_t p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = a.part[(size_t)(sl + u) * a.Vt + t];
#pragma unroll
            for (int u = 0; u < 8; ++u) c += p[u];
        }
        for (; sl < a.S; ++sl) c += a.part[(size_t)sl * a.Vt + t];
        a.counts[t] = c;
    }
    const uint64_t tot = wave_total_u64((uint64_t)c);
    if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = 0;
        for (int w = 0; w < NW; ++w) m += s_w[w];
        if (m) atomicAdd(&a.totals[0], (unsigned long long)m);
    }
}

// One workgroup.  Every pass over the counts takes them in rounds of U * NT
// ids, U loads per thread in flight, thread i of a round holding ids
// base + u * NT + i (coalesced).  Ids are ranked in id order by ballots:
// within a sub-round by the lanes below, across waves and sub-rounds by LDS
// totals, across rounds by a running total.
template <int NT, int U>
__global__ __launch_bounds__(NT) void trim_select_kernel(TrimArgs a) {
    constexpr int NW = NT / kWave;
    __shared__ uint32_t s_n[kTrimDigits];
    __shared__ unsigned long long s_mass[kTrimDigits];
    __shared__ uint32_t s_prefix;
    __shared__ unsigned long long s_above, s_mtot[NW];
    __shared__ uint32_t s_cstar, s_take;
    __shared__ int32_t s_tie, s_mode;     // mode 0: nothing kept, 1: every nonzero id, 2: the cut (c*, tie id)
    __shared__ int32_t s_cnt[U][NW];
    const int32_t Vt = a.Vt;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const unsigned long long valid = a.totals[0], invalid = a.totals[1];
    const double T = (double)a.P * (double)valid;
    if (threadIdx.x == 0) {
        s_prefix = 0;
        s_above = 0;
        s_mode = valid == 0 ? 0 : (T >= (double)valid ? 1 : 2);
        s_cstar = 1;
        s_take = 0;
        s_tie = -1;
    }
    __syncthreads();
    const int mode = s_mode;
    auto load_round = [&](int32_t tb, uint32_t (&c)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t t = tb + u * NT + (int32_t)threadIdx.x;
            c[u] = a.counts[t < Vt ? t : Vt - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (tb + u * NT + (int32_t)threadIdx.x >= Vt) c[u] = 0u;
    };
    if (mode == 2) {
        // the count c* at which the mass from the top reaches T, digit by
        // digit (bits 31..21, 20..10, 9..0): the first bucket from the top
        // whose mass brings the total to T
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int bits = pass == 2 ? 10 : 11;
            const int hi_shift = shift + bits;
            for (int k = threadIdx.x; k < kTrimDigits; k += NT) { s_n[k] = 0; s_mass[k] = 0; }
            __syncthreads();
            const uint32_t pre = s_prefix;
            for (int32_t tb = 0; tb < Vt; tb += U * NT) {
                uint32_t cc[U];
                load_round(tb, cc);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t c = cc[u];
                    bool in = c != 0 && (pass == 0 || (c >> hi_shift) == (pre >> hi_shift));
                    const uint32_t dig = (c >> shift) & ((1u << bits) - 1u);
                    // each wave adds the ids on its leader's digit at once,
                    // twice, then the rest one by one: most counts share
                    // their high digits, and per-lane atomics on one bin
                    // would serialise
                    for (int rep = 0; rep < 2; ++rep) {
                        const uint64_t act = __ballot(in);
                        if (!act) break;
                        const int leader = __ffsll((unsigned long long)act) - 1;
                        const uint32_t dl = (uint32_t)__shfl((int)dig, leader, kWave);
                        const bool mine = in && dig == dl;
                        const uint64_t m = __ballot(mine);
                        const uint64_t mass = wave_total_u64(mine ? (uint64_t)c : 0ull);
                        if (lane == leader) {
                            atomicAdd(&s_n[dl], (uint32_t)__popcll(m));
                            atomicAdd(&s_mass[dl], (unsigned long long)mass);
                        }
                        in = in && !mine;
                    }
                    if (in) {
                        atomicAdd(&s_n[dig], 1u);
                        atomicAdd(&s_mass[dig], (unsigned long long)c);
                    }
                }
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                unsigned long long above = s_above;
                uint32_t sel = 0;
                for (int k = (1 << bits) - 1; k >= 0; --k) {
                    if (s_n[k] == 0) continue;
                    if ((double)(above + s_mass[k]) >= T) { sel = (uint32_t)k; break; }
                    above += s_mass[k];
                }
                s_prefix = pre | (sel << shift);
                s_above = above;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            // the fewest ids of count c* that bring the mass to T (the mass
            // above c* is below T, and all of c*'s ids reach it)
            const uint32_t cs = s_prefix;
            const unsigned long long above = s_above;
            const double need = ceil((T - (double)above) / (double)cs);
            uint32_t take = need < 1.0 ? 1u : (uint32_t)need;
            while (take > 1 && (double)(above + (unsigned long long)(take - 1) * cs) >= T) --take;
            while ((double)(above + (unsigned long long)take * cs) < T) ++take;
            s_cstar = cs;
            s_take = take;
        }
        __syncthreads();
    }
    const uint32_t cstar = s_cstar;
    const int32_t take = (int32_t)s_take;
    // rank of each flagged id in id order: U sub-rounds of NT ids per round
    int32_t run = 0;          // flagged ids in earlier rounds (same in every thread)
    auto rank_round = [&](const bool (&f)[U], int32_t (&rank)[U]) -> int32_t {
        uint64_t bal[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bal[u] = __ballot(f[u]);
            if (lane == 0) s_cnt[u][wv] = (int32_t)__popcll(bal[u]);
        }
        __syncthreads();
        int32_t base = run, total = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int32_t sub = 0, below = 0;
            for (int w = 0; w < NW; ++w) {
                const int32_t n = s_cnt[u][w];
                if (w < wv) below += n;
                sub += n;
            }
            rank[u] = base + below + (int32_t)__popcll(bal[u] & ((1ull << lane) - 1ull));
            base += sub;
            total += sub;
        }
        __syncthreads();
        return total;
    };
    if (mode == 2) {
        // the take-th lowest id of count c*
        for (int32_t tb = 0; tb < Vt; tb += U * NT) {
            uint32_t cc[U];
            load_round(tb, cc);
            bool f[U];
            int32_t rk[U];
#pragma unroll
            for (int u = 0; u < U; ++u) f[u] = cc[u] == cstar;
            const int32_t tot = rank_round(f, rk);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (f[u] && rk[u] == take - 1) s_tie = tb + u * NT + (int32_t)threadIdx.x;
            run += tot;
            if (run >= take) break;                          // uniform: every thread holds run
        }
        __syncthreads();
        run = 0;
    }
    const int32_t tie = s_tie;
    auto kept = [&](uint32_t c, int32_t t) -> bool {
        if (mode == 0 || c == 0) return false;
        if (mode == 1) return true;
        return c > cstar || (c == cstar && t <= tie);
    };
    unsigned long long mass = 0;
    for (int32_t tb = 0; tb < Vt; tb += U * NT) {
        uint32_t cc[U];
        load_round(tb, cc);
        bool f[U];
        int32_t rk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t t = tb + u * NT + (int32_t)threadIdx.x;
            f[u] = t < Vt && kept(cc[u], t);
            if (f[u]) mass += cc[u];
        }
        const int32_t tot = rank_round(f, rk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t t = tb + u * NT + (int32_t)threadIdx.x;
            if (f[u]) a.out_d2t[rk[u]] = t;
            if (a.out_t2d && t < Vt) a.out_t2d[t] = f[u] ? rk[u] : -1;
        }
        run += tot;
    }
    mass = wave_total_u64(mass);
    if (lane == 0) s_mtot[wv] = mass;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long m = 0;
        for (int w = 0; w < NW; ++w) m += s_mtot[w];
        *a.out_vd = run;
        if (a.out_info) {
            a.out_info[0] = (int64_t)m;
            a.out_info[1] = (int64_t)valid;
            a.out_info[2] = (int64_t)invalid;
        }
        a.totals[0] = 0;
        a.totals[1] = 0;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int32_t trim_ranges(int32_t Vt) { return (Vt + kTrimBins - 1) / kTrimBins; }
int32_t trim_slices(int32_t Vt) {
    int32_t s = kTrimTargetWgs / trim_ranges(Vt);
    if (s < 1) s = 1;
    if (s > kTrimMaxSlices) s = kTrimMaxSlices;
    return s;
}
size_t trim_counter_bytes(int32_t Vt) { (void)Vt; return 256; }
size_t trim_data_bytes(int32_t Vt) {
    return align256(sizeof(uint32_t) * (size_t)trim_slices(Vt) * Vt) + align256(sizeof(uint32_t) * (size_t)Vt);
}

hipError_t launch_trim(const TrimArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((trim_part_kernel<kTrimPartThreads, kTrimPartUnroll>),
                       dim3((unsigned)(trim_ranges(a.Vt) * a.S)), dim3(kTrimPartThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((trim_reduce_kernel<256>), dim3((unsigned)((a.Vt + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((trim_select_kernel<kTrimSelThreads, kTrimSelUnroll>), dim3(1), dim3(kTrimSelThreads), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace sv
