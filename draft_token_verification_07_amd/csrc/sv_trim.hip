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
// Two launches:
//   trim_hist_kernel: each workgroup counts a slice of the stream in an LDS
//     hash table (id -> count, open addressing) and adds the table to the
//     global counts with one atomic per distinct id; ids that find no slot
//     within a few probes go straight to the global counts.
//   trim_select_kernel: one workgroup selects the cut exactly in integers: a
//     radix select over the 32-bit counts (8-bit digits, count and mass
//     histograms in LDS) finds the count c* at which the mass from the top
//     reaches P * N and how many ids of count c* are needed, the lowest ids
//     on c* are taken, and a scan over the ids writes d2t and t2d.  It then
//     returns the counts to zero for the next call.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

constexpr int kTrimHistThreads = 512;
constexpr int kTrimSelThreads = 1024;
constexpr int kTrimSlots = 4096;          // LDS hash slots per histogram workgroup
constexpr int kTrimProbes = 8;
constexpr int64_t kTrimSlice = 65536;     // tokens per histogram workgroup

template <int NT>
__global__ __launch_bounds__(NT) void trim_hist_kernel(TrimArgs a) {
    __shared__ int32_t s_id[kTrimSlots];
    __shared__ uint32_t s_cnt[kTrimSlots];
    __shared__ uint32_t s_valid, s_invalid;
    for (int k = threadIdx.x; k < kTrimSlots; k += NT) { s_id[k] = -1; s_cnt[k] = 0; }
    if (threadIdx.x == 0) { s_valid = 0; s_invalid = 0; }
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * kTrimSlice;
    const int64_t i1 = i0 + kTrimSlice < a.N ? i0 + kTrimSlice : a.N;
    uint32_t valid = 0, invalid = 0;
    auto count = [&](int32_t t) {
        if (t < 0 || t >= a.Vt) { ++invalid; return; }
        ++valid;
        int32_t sl = (int32_t)(((uint32_t)t * 0x9E3779B1u) >> 20) & (kTrimSlots - 1);
        for (int p = 0; p < kTrimProbes; ++p) {
            int32_t cur = s_id[sl];
            if (cur == -1) {
                cur = atomicCAS(&s_id[sl], -1, t);
                if (cur == -1) cur = t;
            }
            if (cur == t) {
                atomicAdd(&s_cnt[sl], 1u);
                return;
            }
            sl = (sl + 1) & (kTrimSlots - 1);
        }
        atomicAdd(&a.counts[t], 1u);             // no slot nearby: count it globally
    };
    // four tokens per thread in flight, coalesced across the wave
    for (int64_t i = i0 + threadIdx.x; i < i1; i += 4 * NT) {
        int32_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + u * NT;
            t[u] = a.tokens[j < i1 ? j : i1 - 1];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * NT < i1) count(t[u]);
    }
    atomicAdd(&s_valid, valid);
    atomicAdd(&s_invalid, invalid);
    __syncthreads();
    for (int k = threadIdx.x; k < kTrimSlots; k += NT)
        if (s_id[k] >= 0 && s_cnt[k]) atomicAdd(&a.counts[s_id[k]], s_cnt[k]);
    if (threadIdx.x == 0) {
        if (s_valid) atomicAdd(&a.totals[0], (unsigned long long)s_valid);
        if (s_invalid) atomicAdd(&a.totals[1], (unsigned long long)s_invalid);
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void trim_select_kernel(TrimArgs a) {
    constexpr int NW = NT / kWave;
    __shared__ uint32_t s_n[256];
    __shared__ unsigned long long s_mass[256];
    __shared__ uint32_t s_prefix;
    __shared__ unsigned long long s_above;
    __shared__ uint32_t s_cstar, s_take;
    __shared__ int32_t s_tie, s_wsum[NW];
    __shared__ int32_t s_mode;       // 0: nothing kept, 1: every nonzero id, 2: the cut (c*, tie id)
    const int32_t Vt = a.Vt;
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
    if (mode == 2) {
        // the count c* at which the mass from the top reaches T: digit by digit,
        // the first bucket from the top whose mass brings the total to T
        for (int d = 3; d >= 0; --d) {
            for (int k = threadIdx.x; k < 256; k += NT) { s_n[k] = 0; s_mass[k] = 0; }
            __syncthreads();
            const uint32_t pre = s_prefix;
            const int hi_shift = (d + 1) * 8;
            for (int32_t t = threadIdx.x; t < Vt; t += NT) {
                const uint32_t c = a.counts[t];
                if (c == 0) continue;
                if (d < 3 && (c >> hi_shift) != (pre >> hi_shift)) continue;
                const uint32_t dig = (c >> (d * 8)) & 255u;
                atomicAdd(&s_n[dig], 1u);
                atomicAdd(&s_mass[dig], (unsigned long long)c);
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                unsigned long long above = s_above;
                uint32_t sel = 0;
                for (int k = 255; k >= 0; --k) {
                    if (s_n[k] == 0) continue;
                    if ((double)(above + s_mass[k]) >= T) { sel = (uint32_t)k; break; }
                    above += s_mass[k];
                }
                s_prefix = pre | (sel << (d * 8));
                s_above = above;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            // the fewest ids of count c* that bring the mass to T (the mass
            // above c* is below T, and all of c*'s ids reach it)
            const uint32_t cs = s_prefix;
            const unsigned long long above = s_above;
            double need = ceil((T - (double)above) / (double)cs);
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
    // contiguous id segments per thread
    const int32_t per = (Vt + NT - 1) / NT;
    const int32_t t0 = min(Vt, (int32_t)threadIdx.x * per), t1 = min(Vt, t0 + per);
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    auto excl_scan = [&](int32_t v) -> int32_t {
        const int32_t inc = wave_incl_scan_i32(v);
        if (lane == kWave - 1) s_wsum[wv] = inc;
        __syncthreads();
        int32_t base = inc - v;
        for (int w = 0; w < wv; ++w) base += s_wsum[w];
        __syncthreads();
        return base;
    };
    if (mode == 2) {
        // the take-th lowest id of count c*
        int32_t cnt = 0;
        for (int32_t t = t0; t < t1; ++t) cnt += a.counts[t] == cstar ? 1 : 0;
        const int32_t before = excl_scan(cnt);
        if (before < take && take <= before + cnt) {
            int32_t seen = before;
            for (int32_t t = t0; t < t1; ++t)
                if (a.counts[t] == cstar && ++seen == take) { s_tie = t; break; }
        }
        __syncthreads();
    }
    const int32_t tie = s_tie;
    auto kept = [&](uint32_t c, int32_t t) -> bool {
        if (mode == 0 || c == 0) return false;
        if (mode == 1) return true;
        return c > cstar || (c == cstar && t <= tie);
    };
    int32_t nk = 0;
    unsigned long long mass = 0;
    for (int32_t t = t0; t < t1; ++t) {
        const uint32_t c = a.counts[t];
        if (kept(c, t)) { ++nk; mass += c; }
    }
    int32_t pos = excl_scan(nk);
    for (int32_t t = t0; t < t1; ++t) {
        const uint32_t c = a.counts[t];
        const bool k = kept(c, t);
        if (k) a.out_d2t[pos] = t;
        if (a.out_t2d) a.out_t2d[t] = k ? pos : -1;
        pos += k ? 1 : 0;
        a.counts[t] = 0u;                              // back to zero for the next call
    }
    // totals: the last position is the kept count; the mass by a reduction
    __shared__ unsigned long long s_msum[NW];
    mass = wave_total_u64(mass);
    if (lane == 0) s_msum[wv] = mass;
    __syncthreads();
    if (threadIdx.x == NT - 1) *a.out_vd = pos;
    if (threadIdx.x == 0) {
        unsigned long long m = 0;
        for (int w = 0; w < NW; ++w) m += s_msum[w];
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
size_t trim_counter_bytes(int32_t Vt) { return align256(sizeof(uint32_t) * (size_t)Vt) + 256; }

hipError_t launch_trim(const TrimArgs &a, hipStream_t st) {
    const int64_t grid = a.N > 0 ? (a.N + kTrimSlice - 1) / kTrimSlice : 0;
    if (grid > 0) {
        hipLaunchKernelGGL((trim_hist_kernel<kTrimHistThreads>), dim3((unsigned)grid), dim3(kTrimHistThreads), 0,
                           st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((trim_select_kernel<kTrimSelThreads>), dim3(1), dim3(kTrimSelThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
