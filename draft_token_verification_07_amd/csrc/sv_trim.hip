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
// The kept set is {count > c*} plus the lowest `take` ids of count c*, where
// c* is the largest count whose mass from the top (the count sum of the ids
// of count >= c*) reaches T = P * valid.  Five launches, every one spread
// over the chip; each launch boundary is the only synchronisation, except
// where the last workgroup to arrive on a counter finishes a step:
//   trim_part_kernel: workgroup (r, s) counts the ids t with t % R == r in
//     slice s of the stream (an LDS histogram of ceil(Vt / R) 16-bit bins,
//     two per word; every few rounds the large bins move into per-id
//     overflow counts) and stores the partial histogram.  Ranges by residue
//     spread the frequent ids of a skewed corpus over all ranges.  When S is
//     a multiple of 8 the workgroups of one slice run on one XCD (the block
//     order puts them S apart) and share its L2.  Global atomics only for
//     the rare overflow moves.
//   trim_reduce_kernel: sums the partial histograms and the overflow count
//     of every id (returning the latter to zero), and adds every id to a
//     histogram of count buckets (exact below 128, then 64 per octave; count
//     and mass).  The last workgroup finds the bucket holding c*: the first
//     from the top whose mass brings the total to T.
//   trim_refine_kernel: when that bucket spans several counts, the ids in it
//     give an exact histogram of their counts (buckets up to kTrimFine wide)
//     or a list of them (wider buckets hold counts >= 2^19, so at most
//     2^31 / 2^19 ids), and the last workgroup finds c* and take.
//   trim_count_kernel: per block of kTrimBlock ids, the ids above the cut
//     and on it.
//   trim_write_kernel: every block ranks its kept ids from the block counts
//     before it and writes d2t and t2d; the last block writes the totals.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

constexpr int kTrimPartThreads = 1024;    // one workgroup per CU (its LDS histogram takes 128 KiB)
constexpr int kTrimPartUnroll = 4;        // 16-byte vectors per round (two rounds in flight)
constexpr int kTrimThreads = 256;         // the other launches

// Count bucket of c >= 1: c itself below 128; above, 64 buckets per octave
// [2^e, 2^(e+1)), e = 7..31, by the six bits below the leading one.  The
// bucket index grows with c.
__device__ __forceinline__ int trim_bucket(uint32_t c) {
    if (c < 128u) return (int)c;
    const int e = 31 - __clz(c);
    return 128 + (e - 7) * 64 + (int)((c >> (e - 6)) & 63u);
}
__device__ __forceinline__ void trim_bucket_range(int B, uint32_t *lo, uint32_t *hi) {
    if (B < 128) {
        *lo = *hi = (uint32_t)B;
        return;
    }
    const int e = 7 + (B - 128) / 64, sub = (B - 128) % 64;
    const uint64_t l = (uint64_t)(64 + sub) << (e - 6);
    *lo = (uint32_t)l;
    *hi = (uint32_t)(l + ((uint64_t)1 << (e - 6)) - 1u);
}

__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent_u64(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Adds (number of lanes, sum of val) to `key` for every lane with `in` set:
// the lanes on the leader's key at once (twice), then the rest one by one,
// since most lanes of a skewed input share a few keys and per-lane atomics on
// one address serialise.  Called by every lane of the wave.
template <bool VAL, typename F>
__device__ __forceinline__ void wave_aggregate(bool in, int key, uint64_t val, F &&add) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const uint64_t act = __ballot(in);
        if (!act) return;
        const int leader = __ffsll((unsigned long long)act) - 1;
        const int kl = __shfl(key, leader, kWave);
        const bool mine = in && key == kl;
        const uint64_t m = __ballot(mine);
        uint64_t tot = 0;
        if constexpr (VAL) tot = wave_total_u64(mine ? val : 0ull);
        if (lane == leader) add(kl, (uint32_t)__popcll(m), tot);
        in = in && !mine;
    }
    if (in) add(key, 1u, val);
}

// Exclusive scan of v over the workgroup in thread order; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint64_t wg_excl_scan_u64(uint64_t v, uint64_t *s_tmp, uint64_t *total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const uint64_t inc = wave_incl_scan_u64_dpp(v);
    if (lane == kWave - 1) s_tmp[wv] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint64_t x = s_tmp[w];
        if (w < wv) before += x;
        all += x;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__device__ __forceinline__ uint32_t trim_take(double T, unsigned long long above, uint32_t cs) {
    // the fewest ids of count cs that bring the mass to T (the mass above cs
    // is below T, and all of cs's ids reach it)
    const double need = ceil((T - (double)above) / (double)cs);
    uint32_t take = need < 1.0 ? 1u : (uint32_t)need;
    while (take > 1 && (double)(above + (unsigned long long)(take - 1) * cs) >= T) --take;
    while ((double)(above + (unsigned long long)take * cs) < T) ++take;
    return take;
}

// ---------------------------------------------------------------------------
// Launch 1: partial histograms
// ---------------------------------------------------------------------------
// Bins are 16-bit counters, two to a word (bin k in the low half of word
// k / 2 when k is even), so a range holds twice the ids a 32-bit bin would
// and each token is examined by half as many workgroups.  No bin can wrap:
// every three rounds a sweep moves each bin of kTrimSpill or more into the
// id's overflow count (a global atomic, rare: only ids holding about a sixth
// of a segment get there), and a segment between sweeps adds at most three
// rounds (plus a few unaligned tokens) to a bin.
constexpr uint32_t kTrimSpill = 0x2000u;
constexpr int kTrimSweepRounds = 3;
static_assert((kTrimSpill - 1) + (uint32_t)kTrimSweepRounds * kTrimPartUnroll * kTrimPartThreads * 4 + 8 <= 0xffffu,
              "a 16-bit bin cannot wrap between sweeps");

template <int NT, int U>
__global__ __launch_bounds__(NT) void trim_part_kernel(TrimArgs a) {
    static_assert(NT == kTrimPartThreads && U == kTrimPartUnroll, "the sweep bound assumes this round size");
    __shared__ uint32_t s_h[kTrimBins / 2 + 4];    // bin KB (low half of word KB / 2): the spare below
    const int32_t r = blockIdx.x / a.S, sl = blockIdx.x % a.S;
    const uint32_t Rm = (uint32_t)a.R - 1u, logR = (uint32_t)a.logR;
    const int32_t words = a.KB >> 1;               // KB is a multiple of 8
    for (int k = threadIdx.x; k <= words; k += NT) s_h[k] = 0;
    // what the later launches accumulate into starts at zero
    {
        const int32_t gsz = (int32_t)gridDim.x * NT, gi = (int32_t)blockIdx.x * NT + (int32_t)threadIdx.x;
        for (int32_t k = gi; k < kTrimBuckets; k += gsz) {
            a.hist_n[k] = 0;
            a.hist_m[k] = 0;
        }
        for (int32_t k = gi; k < kTrimFine; k += gsz) a.h2[k] = 0;
    }
    __syncthreads();
    // Ids at or past KB R (negative ones too, as unsigned) are clamped to
    // KB R, whose bin KB in range 0 is a spare that is never stored; ids in
    // [Vt, KB R) land on bins of ids that do not exist, which the reduction
    // skips.  So no token needs a range test of its own, and the invalid
    // tokens are counted as N less the valid ones.
    const uint32_t lim = (uint32_t)a.KB << logR;
    const uint32_t wsh = logR + 1u;                // id -> word
    auto cnt = [&](uint32_t t) {
        const uint32_t u = min(t, lim);
        if ((u & Rm) == (uint32_t)r) {
            // bin u >> logR: word u >> (logR + 1), half (u >> logR) & 1
            const uint32_t half = __builtin_amdgcn_ubfe(u, logR, 1u);
            atomicAdd(&s_h[u >> wsh], half * 0xffffu + 1u);
        }
    };
    // Moves every bin of kTrimSpill or more into its id's overflow count
    // (bins of ids past Vt are just cleared).  Called by the whole workgroup.
    const uint32_t Vt = (uint32_t)a.Vt;
    auto sweep = [&]() {
        lds_barrier();
        for (int k = threadIdx.x; k <= words; k += NT) {
            const uint32_t w = s_h[k];
            if (w & 0xe000e000u) {
                uint32_t f0 = w & 0xffffu, f1 = w >> 16;
                const uint32_t t0 = ((uint32_t)(2 * k) << logR) + (uint32_t)r, t1 = t0 + (1u << logR);
                if (f0 >= kTrimSpill) {
                    if (t0 < Vt) atomicAdd(&a.ovf[t0], f0);
                    f0 = 0;
                }
                if (f1 >= kTrimSpill) {
                    if (t1 < Vt) atomicAdd(&a.ovf[t1], f1);
                    f1 = 0;
                }
                s_h[k] = f0 | (f1 << 16);
            }
        }
        lds_barrier();
    };
    // ok: the token is real
    auto one = [&](int32_t t, bool ok) {
        if (ok) cnt((uint32_t)t);
    };
    const uintptr_t base = reinterpret_cast<uintptr_t>(a.tokens);
    int64_t head = (int64_t)(((16u - (uint32_t)(base & 15u)) & 15u) / 4u);
    if (head > a.N) head = a.N;
    const int64_t nvec = (a.N - head) / 4;
    const int64_t tail0 = head + nvec * 4;
    {
        const bool h = sl == 0 && (int64_t)threadIdx.x < head;
        one(h ? a.tokens[threadIdx.x] : 0, h);
        const bool tl = sl == a.S - 1 && (int64_t)threadIdx.x < a.N - tail0;
        one(tl ? a.tokens[tail0 + threadIdx.x] : 0, tl);
    }
    const u32x4 *body = reinterpret_cast<const u32x4 *>(a.tokens + head);
    const int64_t v0 = nvec * sl / a.S, v1 = nvec * (sl + 1) / a.S;
    // rounds of U * NT vectors; the next round's loads are issued before
    // this round's ids are counted (clamped indices past the slice).  Full
    // rounds count every id; the last, partial round checks its vectors.
    if (v1 > v0) {
        constexpr int64_t step = (int64_t)U * NT;
        auto load = [&](int64_t vb, u32x4 (&raw)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = vb + (int64_t)u * NT + threadIdx.x;
                raw[u] = __builtin_nontemporal_load(&body[j < v1 ? j : v1 - 1]);
            }
        };
        u32x4 cur[U], nxt[U];
        load(v0, cur);
        const int64_t nfull = (v1 - v0) / step;
        int64_t vb = v0;
        for (int64_t it = 0; it < nfull; ++it, vb += step) {
            if (vb + step < v1) load(vb + step, nxt);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                cnt(cur[u].x);
                cnt(cur[u].y);
                cnt(cur[u].z);
                cnt(cur[u].w);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            if ((it + 1) % kTrimSweepRounds == 0 && vb + step < v1) sweep();
        }
        if (vb < v1) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = vb + (int64_t)u * NT + threadIdx.x < v1;
                one((int32_t)cur[u].x, ok);
                one((int32_t)cur[u].y, ok);
                one((int32_t)cur[u].z, ok);
                one((int32_t)cur[u].w, ok);
            }
        }
    }
    __syncthreads();
    uint32_t *dst = a.part + ((size_t)sl * a.R + r) * words;
    for (int k = threadIdx.x; k < words; k += NT) dst[k] = s_h[k];
}

// ---------------------------------------------------------------------------
// Launch 2: counts, the count-bucket histogram, the boundary bucket
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void trim_boundary(const TrimArgs &a) {
    constexpr int PER = (kTrimBuckets + NT - 1) / NT;
    __shared__ unsigned long long s_tot[2];
    __shared__ uint64_t s_tmp[NT / kWave];
    __shared__ int s_B;
    __shared__ unsigned long long s_aboveB;
    if (threadIdx.x == 0) {
        s_tot[0] = ld_agent_u64(&a.totals[0]);
        // every token is valid (an id in [0, Vt)) or invalid
        s_tot[1] = (unsigned long long)a.N - s_tot[0];
        // the counter region goes back to zero (read by this workgroup only)
        __hip_atomic_store(&a.totals[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_B = -1;
        s_aboveB = 0;
    }
    __syncthreads();
    const unsigned long long valid = s_tot[0], invalid = s_tot[1];
    const double T = (double)a.P * (double)valid;
    const int mode = valid == 0 ? 0 : (T >= (double)valid ? 1 : 2);
    if (mode == 2) {
        // thread i takes buckets [top - PER (i + 1), top - PER i): chunk sums,
        // the mass above each chunk, then the crossing chunk walks its buckets.
        // The masses are loaded in one round (unconditionally, at clamped
        // indices) and kept for the walk.
        const int hiB = kTrimBuckets - 1 - PER * (int)threadIdx.x;
        unsigned long long mb[PER];
        uint64_t m = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const unsigned long long v = ld_agent_u64(&a.hist_m[max(hiB - q, 0)]);
            mb[q] = hiB - q >= 0 ? v : 0ull;
            m += mb[q];
        }
        uint64_t all;
        const uint64_t before = wg_excl_scan_u64<NT>(m, s_tmp, &all);
        if ((double)before < T && (double)(before + m) >= T) {
            unsigned long long acc = before;
            bool found = false;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                if (found || hiB - q < 0 || mb[q] == 0) continue;
                if ((double)(acc + mb[q]) >= T) {
                    s_B = hiB - q;
                    s_aboveB = acc;
                    found = true;
                } else {
                    acc += mb[q];
                }
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        TrimState st;
        st.valid = valid;
        st.invalid = invalid;
        st.T = T;
        st.mode = mode;
        st.aboveB = 0;
        st.above = 0;
        st.refine = 0;
        st.lo = st.hi = 1;
        st.nB = 0;
        st.cstar = 1;
        st.take = 0;
        st.list_n = 0;
        const int B = s_B;
        if (mode == 2 && B >= 0) {
            uint32_t lo, hi;
            trim_bucket_range(B, &lo, &hi);
            st.lo = lo;
            st.hi = hi;
            st.aboveB = s_aboveB;
            st.nB = ld_agent_u32(&a.hist_n[B]);
            if (lo == hi) {
                st.cstar = lo;
                st.above = s_aboveB;
                st.take = trim_take(T, s_aboveB, lo);
            } else {
                st.refine = (uint64_t)hi - lo + 1 <= (uint64_t)kTrimFine ? 1 : 2;
            }
        }
        *a.state = st;
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void trim_reduce_kernel(TrimArgs a) {
    constexpr int NW = NT / kWave;
    __shared__ uint64_t s_w[NW];
    __shared__ int s_last;
    __shared__ uint32_t s_hn[kTrimBuckets];
    __shared__ unsigned long long s_hm[kTrimBuckets];
    for (int b = threadIdx.x; b < kTrimBuckets; b += NT) {
        s_hn[b] = 0;
        s_hm[b] = 0;
    }
    __syncthreads();
    // thread: bins k0..k0+3 of range r (one 8-byte load of two words per
    // slice, kTrimRedBatch slices in flight; rows of KB / 2 words, KB a
    // multiple of 8), i.e. ids (k0 + q) R + r, plus their overflow counts
    constexpr int kTrimRedBatch = 16;
    const int32_t i = (int32_t)blockIdx.x * NT + (int32_t)threadIdx.x;      // over [0, R * KB / 4)
    const int32_t q4 = a.KB >> 2;
    const int32_t r = i / q4, k0 = (i - r * q4) << 2;
    const bool own = r < a.R;
    u32x4 c4 = {0u, 0u, 0u, 0u};
    // the ids' overflow counts, loaded first so that their latency hides
    // under the slices' loads
    // (unconditional loads at clamped ids, used only for ids this thread
    // owns: a load under a divergent branch is waited for inside it)
    uint32_t ov[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ov[q] = a.ovf[min(max(((k0 + q) << a.logR) + r, 0), a.Vt - 1)];
    if (own) {
        const int32_t words = a.KB >> 1;
        const uint2 *p = reinterpret_cast<const uint2 *>(a.part + (size_t)r * words + (k0 >> 1));
        const size_t stride = ((size_t)a.R * words) >> 1;
        auto add = [&](const uint2 &w) {
            c4.x += w.x & 0xffffu; c4.y += w.x >> 16; c4.z += w.y & 0xffffu; c4.w += w.y >> 16;
        };
        int32_t sl = 0;
        for (; sl + kTrimRedBatch <= a.S; sl += kTrimRedBatch) {
            uint2 q[kTrimRedBatch];
#pragma unroll
            for (int u = 0; u < kTrimRedBatch; ++u) q[u] = p[(size_t)(sl + u) * stride];
#pragma unroll
            for (int u = 0; u < kTrimRedBatch; ++u) add(q[u]);
        }
        for (; sl < a.S; ++sl) add(p[(size_t)sl * stride]);
    }
    // the workgroup's bucket histogram in LDS, then one global add per
    // nonzero bucket (a bucket of small counts holds most ids of a skewed
    // corpus, and per-id global atomics on it would serialise)
    uint64_t csum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int32_t t = ((k0 + q) << a.logR) + r;
        uint32_t c = q == 0 ? c4.x : q == 1 ? c4.y : q == 2 ? c4.z : c4.w;
        if (own && t < a.Vt) {
            // the overflow count goes back to zero for the next call
            const uint32_t o = ov[q];
            if (o) {
                c += o;
                a.ovf[t] = 0;
            }
            a.counts[t] = c;
            csum += c;
            if (c > 0) {
                const int b = trim_bucket(c);
                atomicAdd(&s_hn[b], 1u);
                atomicAdd(&s_hm[b], (unsigned long long)c);
            }
        }
    }
    const uint64_t tot = wave_total_u64(csum);
    if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = tot;
    __syncthreads();
    for (int b = threadIdx.x; b < kTrimBuckets; b += NT) {
        const uint32_t n = s_hn[b];
        if (n) {
            atomicAdd(&a.hist_n[b], n);
            atomicAdd(&a.hist_m[b], s_hm[b]);
        }
    }
    if (threadIdx.x == 0) {
        uint64_t m = 0;
        for (int w = 0; w < NW; ++w) m += s_w[w];
        if (m) atomicAdd(&a.totals[0], (unsigned long long)m);
    }
    if (!arrive_last(&a.arrive[0], gridDim.x, &s_last)) return;
    trim_boundary<NT>(a);
}

// ---------------------------------------------------------------------------
// Launch 3: the exact cut inside the boundary bucket
// ---------------------------------------------------------------------------
// The fields it needs are read from the state one by one (uniform loads):
// a copy of the whole struct is kept in per-thread memory by the compiler.
template <int NT>
__device__ __forceinline__ void trim_cut(const TrimArgs &a) {
    __shared__ uint64_t s_tmp[NT / kWave];
    __shared__ uint32_t s_cs;
    __shared__ unsigned long long s_above;
    __shared__ uint64_t s_l[kTrimList];
    const TrimState *sp = a.state;
    const double T = sp->T;
    const unsigned long long aboveB = sp->aboveB;
    const uint32_t lo = sp->lo, hi = sp->hi;
    if (threadIdx.x == 0) {
        s_cs = 0;
        s_above = aboveB;
    }
    __syncthreads();
    if (sp->refine == 1) {
        // exact histogram over [lo, hi]: thread i takes the values
        // (hi - PER (i + 1), hi - PER i]
        constexpr int PER = (kTrimFine + NT - 1) / NT;
        const int64_t top = (int64_t)hi - (int64_t)PER * threadIdx.x;
        // the masses v * (ids of count v), loaded in one round (clamped
        // indices) and kept for the walk
        unsigned long long mv[PER];
        uint64_t m = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int64_t v = top - q;
            const uint32_t n = ld_agent_u32(&a.h2[v >= (int64_t)lo ? v - lo : 0]);
            mv[q] = v >= (int64_t)lo ? (unsigned long long)v * n : 0ull;
            m += mv[q];
        }
        uint64_t all;
        const uint64_t before = aboveB + wg_excl_scan_u64<NT>(m, s_tmp, &all);
        if ((double)before < T && (double)(before + m) >= T) {
            unsigned long long acc = before;
            bool found = false;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                if (found || mv[q] == 0) continue;
                if ((double)(acc + mv[q]) >= T) {
                    s_cs = (uint32_t)(top - q);
                    s_above = acc;
                    found = true;
                } else {
                    acc += mv[q];
                }
            }
        }
        __syncthreads();
    } else {
        // the bucket's counts, sorted: c* is the largest count whose mass
        // from the top reaches T
        const int32_t L = min((int32_t)ld_agent_u32(&a.state->list_n), kTrimList);
        const int P = pow2_at_least(L > 1 ? L : 2);
        for (int q = threadIdx.x; q < P; q += NT) s_l[q] = q < L ? (uint64_t)ld_agent_u32(&a.list[q]) : 0ull;
        bitonic_sort_u64<NT>(s_l, P);                          // ascending; ends with a barrier
        // the j-th largest is s_l[P - 1 - j]; thread i takes j in [PJ i, PJ (i + 1))
        const int PJ = (P + NT - 1) / NT;
        uint64_t m = 0;
        for (int q = 0; q < PJ; ++q) {
            const int j = PJ * (int)threadIdx.x + q;
            if (j < P) m += s_l[P - 1 - j];
        }
        uint64_t all;
        const uint64_t before = aboveB + wg_excl_scan_u64<NT>(m, s_tmp, &all);
        if ((double)before < T && (double)(before + m) >= T) {
            unsigned long long acc = before;
            for (int q = 0; q < PJ; ++q) {
                const int j = PJ * (int)threadIdx.x + q;
                if (j >= P) break;
                const uint64_t v = s_l[P - 1 - j];
                if ((double)(acc + v) >= T) {
                    s_cs = (uint32_t)v;
                    break;
                }
                acc += v;
            }
        }
        __syncthreads();
        // the mass strictly above c* (entries equal to c* may come before the crossing)
        const uint32_t cs = s_cs;
        uint64_t mg = 0;
        for (int q = threadIdx.x; q < P; q += NT)
            if (s_l[q] > cs) mg += s_l[q];
        uint64_t g;
        (void)wg_excl_scan_u64<NT>(mg, s_tmp, &g);
        if (threadIdx.x == 0) s_above = aboveB + g;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const uint32_t cs = s_cs > 0 ? s_cs : lo;             // found by construction
        const unsigned long long above = s_above;
        a.state->cstar = cs;
        a.state->above = above;
        a.state->take = trim_take(T, above, cs);
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void trim_refine_kernel(TrimArgs a) {
    __shared__ int s_last;
    // Alike in every workgroup (none then arrives).  The fields are read on
    // their own, as uniform loads: a copy of the whole state per thread cost
    // ~7 us even for the common cut that needs no refining.
    const int32_t refine = a.state->refine;
    if (a.state->mode != 2 || refine == 0) return;
    const uint32_t lo = a.state->lo, hi = a.state->hi;
    const int32_t t0 = ((int32_t)blockIdx.x * NT + (int32_t)threadIdx.x) * 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int32_t t = t0 + u;
        const uint32_t c = t < a.Vt ? a.counts[t] : 0u;
        const bool in = c >= lo && c <= hi && c > 0;
        if (refine == 1) {
            wave_aggregate<false>(in, (int)(c - lo), 0ull,
                                  [&](int k, uint32_t n, uint64_t) { atomicAdd(&a.h2[k], n); });
        } else {
            // published for the last workgroup, which may run on another XCD
            const int32_t pos = wave_append(in, reinterpret_cast<int32_t *>(&a.state->list_n));
            if (in && pos < kTrimList) __hip_atomic_store(&a.list[pos], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (!arrive_last(&a.arrive[1], gridDim.x, &s_last)) return;
    trim_cut<NT>(a);
}

// ---------------------------------------------------------------------------
// Launches 4 and 5: block counts, then d2t / t2d
// ---------------------------------------------------------------------------
struct TrimCut {
    int mode;
    uint32_t cstar;
    __device__ __forceinline__ bool def(uint32_t c) const { return mode == 1 ? c > 0 : (mode == 2 && c > cstar); }
    __device__ __forceinline__ bool tie(uint32_t c) const { return mode == 2 && c == cstar; }
};

template <int NT>
__global__ __launch_bounds__(NT) void trim_count_kernel(TrimArgs a) {
    static_assert(NT * 4 == kTrimBlock, "four ids per thread");
    __shared__ uint64_t s_tmp[NT / kWave];
    const TrimState st = *a.state;
    const TrimCut cut{st.mode, st.cstar};
    const int32_t t0 = (int32_t)blockIdx.x * kTrimBlock + (int32_t)threadIdx.x * 4;
    uint32_t nd = 0, nt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int32_t t = t0 + u;
        const uint32_t c = t < a.Vt ? a.counts[t] : 0u;
        nd += cut.def(c) ? 1u : 0u;
        nt += cut.tie(c) ? 1u : 0u;
    }
    uint64_t tot;
    (void)wg_excl_scan_u64<NT>(((uint64_t)nd << 32) | nt, s_tmp, &tot);
    if (threadIdx.x == 0) {
        a.blockdef[blockIdx.x] = (uint32_t)(tot >> 32);
        a.blocktie[blockIdx.x] = (uint32_t)tot;
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void trim_write_kernel(TrimArgs a) {
    static_assert(NT * 4 == kTrimBlock, "four ids per thread");
    __shared__ uint64_t s_tmp[NT / kWave];
    const TrimState st = *a.state;
    const TrimCut cut{st.mode, st.cstar};
    const uint32_t take = st.mode == 2 ? st.take : 0u;
    const int32_t j = blockIdx.x;
    // ids above the cut and on it in the blocks before this one
    uint64_t pre = 0;
    for (int32_t q = threadIdx.x; q < j; q += NT) pre += ((uint64_t)a.blockdef[q] << 32) | a.blocktie[q];
    uint64_t before;
    (void)wg_excl_scan_u64<NT>(pre, s_tmp, &before);
    const int32_t t0 = j * kTrimBlock + (int32_t)threadIdx.x * 4;
    uint32_t c[4], nd = 0, nt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int32_t t = t0 + u;
        c[u] = t < a.Vt ? a.counts[t] : 0u;
        nd += cut.def(c[u]) ? 1u : 0u;
        nt += cut.tie(c[u]) ? 1u : 0u;
    }
    uint64_t blk;
    const uint64_t ex = wg_excl_scan_u64<NT>(((uint64_t)nd << 32) | nt, s_tmp, &blk);
    uint32_t rd = (uint32_t)(before >> 32) + (uint32_t)(ex >> 32);     // ids above the cut before t
    uint32_t rt = (uint32_t)before + (uint32_t)ex;                     // ids on the cut before t
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int32_t t = t0 + u;
        if (t >= a.Vt) break;
        const bool d = cut.def(c[u]), e = cut.tie(c[u]);
        const bool kept = d || (e && rt < take);
        const uint32_t pos = rd + (rt < take ? rt : take);
        if (kept) a.out_d2t[pos] = t;
        if (a.out_t2d) a.out_t2d[t] = kept ? (int32_t)pos : -1;
        rd += d ? 1u : 0u;
        rt += e ? 1u : 0u;
    }
    if (j == a.nblocks - 1 && threadIdx.x == 0) {
        const uint32_t nd_all = (uint32_t)(before >> 32) + (uint32_t)(blk >> 32);
        const uint32_t nt_all = (uint32_t)before + (uint32_t)blk;
        *a.out_vd = (int32_t)(nd_all + (nt_all < take ? nt_all : take));
        if (a.out_info) {
            const unsigned long long mass =
                st.mode == 2 ? st.above + (unsigned long long)take * st.cstar : (st.mode == 1 ? st.valid : 0ull);
            a.out_info[0] = (int64_t)mass;
            a.out_info[1] = (int64_t)st.valid;
            a.out_info[2] = (int64_t)st.invalid;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

hipError_t launch_trim(const TrimArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((trim_part_kernel<kTrimPartThreads, kTrimPartUnroll>), dim3((unsigned)(a.R * a.S)),
                       dim3(kTrimPartThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nred = ((int64_t)a.R * (a.KB / 4) + kTrimThreads - 1) / kTrimThreads;
    hipLaunchKernelGGL((trim_reduce_kernel<kTrimThreads>), dim3((unsigned)nred), dim3(kTrimThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((trim_refine_kernel<kTrimThreads>), dim3((unsigned)a.nblocks), dim3(kTrimThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((trim_count_kernel<kTrimThreads>), dim3((unsigned)a.nblocks), dim3(kTrimThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((trim_write_kernel<kTrimThreads>), dim3((unsigned)a.nblocks), dim3(kTrimThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
