// sv_rows.h -- device helpers over logits rows shared by the sampling kernels
// (verification and the draft-side sampler): row descriptors and kept-set
// tests, workgroup scans and sorts, DPP wave reductions, LDS appends, the
// fixed-point weight codes, the exact whole-row top-p select and the
// whole-row inverse-CDF draw.
#pragma once

#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

// Rarely taken paths (exact whole-row select, wide-band radix, whole-row
// draw).  SV_RARE_OUTLINE keeps them out of line so the common path stays
// compact in the instruction cache; inlined otherwise.
#ifdef SV_RARE_OUTLINE
#define SV_RARE __attribute__((noinline))
#else
#define SV_RARE __forceinline__
#endif

// ---------------------------------------------------------------------------
// Row descriptors
// ---------------------------------------------------------------------------

// Key of a logit for ordering; -0 is folded onto +0 so that equal values
// share a key (the stable sort of the page compares values).
__device__ __forceinline__ uint32_t zkey(float z) { return fkey(z + 0.0f); }

__device__ __forceinline__ bool row_kept(const RowDesc &d, float z, int32_t j) {
    const uint32_t k = zkey(z);
    return k > d.key || (k == d.key && j <= d.tie_cut);
}

// p(j) of a row: w / Zk on kept ids, 0 elsewhere and on rows without mass.
__device__ __forceinline__ float row_prob(const RowDesc &d, float z, int32_t j, float c) {
    if ((d.flags & RD_NO_MASS) || !row_kept(d, z, j)) return 0.0f;
    return exp2_hw((z - d.m) * c) / d.Zk;
}

// A descriptor read field by field (a whole-struct copy through a
// conditional would be staged in private memory).
__device__ __forceinline__ RowDesc load_desc(const RowDesc *p) {
    RowDesc d;
    d.m = p->m;
    d.Z = p->Z;
    d.Zk = p->Zk;
    d.key = p->key;
    d.tie_cut = p->tie_cut;
    d.nkept = p->nkept;
    d.flags = p->flags;
    d.ptok = p->ptok;
    return d;
}

__device__ __forceinline__ bool bad_max(float m) { return !(m > -INFINITY) || m == INFINITY; }

template <int DT>
__device__ __forceinline__ float ld_logit(const void *base, int64_t i) {
    return Elem<DT>::load(base, i);
}

// first j in [0, n) with d2t[j] >= t (d2t ascending)
__device__ __forceinline__ int32_t lower_bound_i32(const int32_t *v, int32_t n, int32_t t) {
    int32_t lo = 0, hi = n;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (v[mid] < t) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Workgroup primitives (all threads must call them)
// ---------------------------------------------------------------------------

template <int NT>
__device__ __forceinline__ int32_t wg_min_i32(int32_t v, int32_t *s_tmp) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const int32_t w = __shfl_xor(v, o, kWave);
        v = w < v ? w : v;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = v;
    __syncthreads();
    int32_t t = s_tmp[0];
    for (int w = 1; w < NT / kWave; ++w) t = s_tmp[w] < t ? s_tmp[w] : t;
    __syncthreads();
    return t;
}

template <int NT>
__device__ __forceinline__ int32_t wg_max_i32(int32_t v, int32_t *s_tmp) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const int32_t w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = v;
    __syncthreads();
    int32_t t = s_tmp[0];
    for (int w = 1; w < NT / kWave; ++w) t = s_tmp[w] > t ? s_tmp[w] : t;
    __syncthreads();
    return t;
}

// Exclusive scan of one double per thread in thread order; *total gets the sum.
template <int NT>
__device__ __forceinline__ double wg_excl_scan_f64(double v, double *s_tmp, double *total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const double inc = wave_incl_scan(v);
    double exc = __shfl_up(inc, 1, kWave);
    if (lane == 0) exc = 0.0;
    if (lane == kWave - 1) s_tmp[w] = inc;
    __syncthreads();
    double base = 0.0, tot = 0.0;
    for (int k = 0; k < NT / kWave; ++k) {
        if (k < w) base += s_tmp[k];
        tot += s_tmp[k];
    }
    __syncthreads();
    *total = tot;
    return base + exc;
}

// Ascending bitonic sort of P (a power of two) 64-bit keys in LDS.
template <int NT>
__device__ __forceinline__ void bitonic_sort_u64(uint64_t *s, int P) {
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < P; i += NT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t x = s[i], y = s[ixj];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) { s[i] = y; s[ixj] = x; }
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Inverse-CDF search over n weights given in id order by get(s) -> (weight).
// Each thread owns a contiguous segment; sums are float64 in index order.
// Returns the first s with inclusive sum > target, else the last s with a
// positive weight, else -1.  *total receives the sum of all weights.
template <int NT, typename G>
__device__ __forceinline__ int32_t wg_inverse_cdf(int32_t n, G &&get, double u, bool u_is_fraction, double *s_dtmp,
                                  int32_t *s_itmp, double *total_out) {
    const int32_t per = (n + NT - 1) / NT;
    const int32_t s0 = min(n, (int32_t)threadIdx.x * per), s1 = min(n, s0 + per);
    double seg = 0.0;
    for (int32_t s = s0; s < s1; ++s) seg += (double)get(s);
    double total;
    const double base = wg_excl_scan_f64<NT>(seg, s_dtmp, &total);
    *total_out = total;
    const double target = u_is_fraction ? u * total : u;
    int32_t found = INT32_MAX, lastpos = -1;
    double run = base;
    for (int32_t s = s0; s < s1; ++s) {
        const float w = get(s);
        if (w > 0.0f) lastpos = s;
        run += (double)w;
        if (run > target) { found = s; break; }
    }
    // lastpos of this segment matters only when nobody found a crossing
    if (found == INT32_MAX) {
        for (int32_t s = s1 - 1; s >= s0 && lastpos < 0; --s)
            if (get(s) > 0.0f) lastpos = s;
    }
    const int32_t f = wg_min_i32<NT>(found, s_itmp);
    if (f != INT32_MAX) return f;
    return wg_max_i32<NT>(lastpos, s_itmp);
}

// ---------------------------------------------------------------------------
// Draws over whole target rows (no kept list): the residual max(0, p_n - q_n),
// or p itself, over the target ids in tiles.  A tile's weights are staged in
// LDS in id order; each thread owns a contiguous segment of them; segment sums
// (float64, in id order) are scanned in thread order, and the tile's mass is
// that scan's total.  The pass that picks a tile and the pass that searches
// inside it compute the same numbers the same way, so they agree bit for bit.
// ---------------------------------------------------------------------------
struct DrawCtx {
    const void *trow;          // target row n
    const void *drow;          // draft row n (residual only)
    const int32_t *d2t;        // draft id -> target id, or null
    int32_t Vd;
    RowDesc dp, dq;
    float c;
    bool resid;
};

// First index in [0, n) whose value is >= t in the ascending array v, found
// by one whole wave: 64 probes narrow the range 64-fold per round (three
// dependent loads for 32000 entries, where a binary search takes fifteen).
// All 64 lanes call it together and get the same value.
__device__ __forceinline__ int32_t wave_lower_bound(const int32_t *v, int32_t n, int32_t t) {
    const int lane = threadIdx.x & (kWave - 1);
    int32_t lo = 0, hi = n;                       // the answer lies in [lo, hi]
    while (hi - lo > kWave) {
        const int32_t step = (hi - lo + kWave - 1) / kWave;
        const int32_t i = lo + lane * step;
        const int cnt = __popcll(__ballot(i < hi && v[i] < t));
        if (cnt == 0) {
            hi = lo;
            break;
        }
        const int32_t nlo = lo + (cnt - 1) * step + 1;
        hi = min(hi, lo + cnt * step);
        lo = nlo;
    }
    const int32_t i = lo + lane;
    return lo + __popcll(__ballot(i < hi && v[i] < t));
}

// The same search by groups of G consecutive lanes (G divides 64), each group
// with its own t: G probes per round narrow a group's range G-fold, so one
// wave runs 64 / G searches at once.  Every lane of a group returns the
// group's answer; all 64 lanes call it together.
template <int G>
__device__ __forceinline__ int32_t group_lower_bound(const int32_t *v, int32_t n, int32_t t) {
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const uint64_t gmask = (G == kWave ? ~0ull : ((1ull << (G & (kWave - 1))) - 1ull)) << (lane & ~(G - 1));
    int32_t lo = 0, hi = n;                       // the group's answer lies in [lo, hi]
    while (__ballot(hi - lo > G)) {
        const bool active = hi - lo > G;
        const int32_t step = active ? (hi - lo + G - 1) / G : 0;
        const int32_t i = lo + gl * step;
        const int cnt = __popcll(__ballot(active && i < hi && v[i] < t) & gmask);
        if (active) {
            if (cnt == 0) {
                hi = lo;
            } else {
                const int32_t nlo = lo + (cnt - 1) * step + 1;
                hi = min(hi, lo + cnt * step);
                lo = nlo;
            }
        }
    }
    const int32_t i = lo + gl;
    return lo + __popcll(__ballot(i < hi && v[i] < t) & gmask);
}

// The draft ids whose d2t entries fall in target ids [t0, t1): [s_j[0], s_j[1]).
// Waves 0 and 1 search in parallel (NT >= 128).
template <int NT>
__device__ __forceinline__ void tile_jrange(const DrawCtx &x, int32_t t0, int32_t t1, int32_t *s_j) {
    static_assert(NT >= 2 * kWave, "two waves search the two ends");
    const int w = threadIdx.x / kWave;
    if (w < 2) {
        const int32_t j = wave_lower_bound(x.d2t, x.Vd, w == 0 ? t0 : t1);
        if ((threadIdx.x & (kWave - 1)) == 0) s_j[w] = j;
    }
    __syncthreads();
}

// Weights of target ids [t0, t0 + len) into s_w[0, len), len <= kTile.
// [j0, j1) are the draft ids mapped into the tile (d2t residual only).  Every
// load of the tile is issued before any is used (one round trip); the q
// values of mapped ids are scattered into s_w, then each slot is overwritten
// with its weight by the thread that reads it.
template <int DTT, int DTD, int NT>
__device__ __forceinline__ void tile_fill(const DrawCtx &x, int32_t t0, int32_t len, int32_t j0, int32_t j1,
                                          float *s_w) {
    // These whole-row draws are rare paths: plain loops that keep few
    // registers live (the kernels they sit in are sized for their hot paths).
    const bool scat = x.resid && x.d2t != nullptr && j1 > j0;
    const bool dense_q = x.resid && x.d2t == nullptr;
    if (scat) {
        for (int32_t k = threadIdx.x; k < len; k += NT) s_w[k] = 0.0f;
        __syncthreads();
        for (int32_t j = j0 + (int32_t)threadIdx.x; j < j1; j += NT) {
            const int32_t k = x.d2t[j] - t0;
            if ((uint32_t)k < (uint32_t)len) s_w[k] = row_prob(x.dq, ld_logit<DTD>(x.drow, j), j, x.c);
        }
        __syncthreads();
    }
    for (int32_t k = threadIdx.x; k < len; k += NT) {
        float r = row_prob(x.dp, ld_logit<DTT>(x.trow, t0 + k), t0 + k, x.c);
        if (x.resid) {
            // q: scattered from the mapped draft ids, or the same id's draft logit
            const float q = scat ? s_w[k] : dense_q ? row_prob(x.dq, ld_logit<DTD>(x.drow, t0 + k), t0 + k, x.c) : 0.0f;
            r = r - q > 0.0f ? r - q : 0.0f;
        }
        s_w[k] = r;
    }
    __syncthreads();
}

// This thread's segment [*s0, *s1) of a filled tile and its float64 sum in id order.
template <int NT>
__device__ __forceinline__ double tile_seg(const float *s_w, int32_t len, int32_t *s0, int32_t *s1) {
    const int32_t per = (len + NT - 1) / NT;
    *s0 = min(len, (int32_t)threadIdx.x * per);
    *s1 = min(len, *s0 + per);
    double seg = 0.0;
    for (int32_t s = *s0; s < *s1; ++s) seg += (double)s_w[s];
    return seg;
}

// Exclusive (*lo) and inclusive (*hi) prefix of one float64 per thread, in
// thread order, and the total.  hi of thread t equals lo of thread t + 1 bit
// for bit, and hi of the last thread equals the total.
template <int NT>
__device__ __forceinline__ void wg_scan_f64(double v, double *s_tmp, double *lo, double *hi, double *total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const double inc = wave_incl_scan(v);
    double exc = __shfl_up(inc, 1, kWave);
    if (lane == 0) exc = 0.0;
    if (lane == kWave - 1) s_tmp[w] = inc;
    __syncthreads();
    double base = 0.0, tot = 0.0;
    for (int k = 0; k < NT / kWave; ++k) {
        if (k < w) base += s_tmp[k];
        tot += s_tmp[k];
    }
    __syncthreads();
    *lo = base + exc;
    *hi = base + inc;
    *total = tot;
}

// Mass of a filled tile (the same numbers tile_search scans).
template <int NT>
__device__ __forceinline__ double tile_total(const float *s_w, int32_t len, double *s_dtmp) {
    int32_t s0, s1;
    const double seg = tile_seg<NT>(s_w, len, &s0, &s1);
    double lo, hi, tot;
    wg_scan_f64<NT>(seg, s_dtmp, &lo, &hi, &tot);
    return tot;
}

// Offset in a filled tile of the first id of positive weight whose inclusive
// sum exceeds tin (0 <= tin < the tile's mass); the tile's last id of positive
// weight when rounding leaves none; -1 when every weight is zero.
template <int NT>
__device__ __forceinline__ int32_t tile_search(const float *s_w, int32_t len, double tin, double *s_dtmp,
                                               int32_t *s_itmp) {
    int32_t s0, s1;
    const double seg = tile_seg<NT>(s_w, len, &s0, &s1);
    double lo, hi, tot;
    wg_scan_f64<NT>(seg, s_dtmp, &lo, &hi, &tot);
    int32_t found = INT32_MAX;
    if (lo <= tin && tin < hi) {               // one thread's segment brackets tin
        double run = lo;
        int32_t lastpos = -1;
        for (int32_t s = s0; s < s1; ++s) {
            const float w = s_w[s];
            if (w > 0.0f) {
                lastpos = s;
                run += (double)w;
                if (run > tin) {
                    found = s;
                    break;
                }
            }
        }
        if (found == INT32_MAX) found = lastpos;
    }
    const int32_t f = wg_min_i32<NT>(found, s_itmp);
    if (f != INT32_MAX) return f;
    int32_t lp = -1;
    for (int32_t s = s1 - 1; s >= s0; --s)
        if (s_w[s] > 0.0f) {
            lp = s;
            break;
        }
    return wg_max_i32<NT>(lp, s_itmp);
}

// A whole draw in one workgroup (rare paths): one sweep over the tiles sums
// the masses, a second finds the tile holding u * S and searches it.
// Returns -1 when S == 0.
template <int DTT, int DTD, int NT>
__device__ SV_RARE int32_t draw_row_one_wg(const DrawCtx &x, int32_t Vt, int32_t tile, double u, float *s_w,
                                           double *s_dtmp, int32_t *s_itmp, int32_t *s_j) {
    auto fill = [&](int32_t t0, int32_t len) {
        int32_t j0 = 0, j1 = 0;
        if (x.resid && x.d2t) {
            tile_jrange<NT>(x, t0, t0 + len, s_j);
            j0 = s_j[0];
            j1 = s_j[1];
        }
        tile_fill<DTT, DTD, NT>(x, t0, len, j0, j1, s_w);
    };
    double S = 0.0;
    for (int32_t t0 = 0; t0 < Vt; t0 += tile) {
        const int32_t len = min(tile, Vt - t0);
        fill(t0, len);
        S += tile_total<NT>(s_w, len, s_dtmp);
    }
    if (!(S > 0.0)) return -1;
    const double target = u * S;                // < S for u < 1
    double run = 0.0;
    for (int32_t t0 = 0; t0 < Vt; t0 += tile) {
        const int32_t len = min(tile, Vt - t0);
        fill(t0, len);
        const double m = tile_total<NT>(s_w, len, s_dtmp);
        if (m > 0.0 && target < run + m) {
            const int32_t k = tile_search<NT>(s_w, len, target - run, s_dtmp, s_itmp);
            return k < 0 ? -1 : t0 + k;
        }
        run += m;
    }
    return -1;
}

// ---------------------------------------------------------------------------
// Top-p rows: exact radix select over the whole row (fallback path).
// Finds the boundary key by mass with 8-bit digits of the 32-bit key, in
// fixed point (deterministic integer sums), then the tie cut by id, then the
// kept list when it fits.
// ---------------------------------------------------------------------------
constexpr double kFix = 274877906944.0;   // 2^38: w in (0, 1] -> fixed point; 2^24 ids fit in 2^62

template <int DT, int NT, bool LIST = true>
__device__ SV_RARE void topp_exact_row(const void *row, int32_t L, float m, float c, float top_p,
                               RowDesc *out, KeptEnt *kept, unsigned char *lds) {
    uint32_t *s_cnt = reinterpret_cast<uint32_t *>(lds);                       // [256]
    unsigned long long *s_mass = reinterpret_cast<unsigned long long *>(lds + 1024);  // [256]
    __shared__ uint32_t s_prefix, s_cnt_above, s_g;
    __shared__ unsigned long long s_mabove, s_T0, s_total;
    __shared__ int32_t s_tie_cut, s_nlist;

    if (threadIdx.x == 0) { s_prefix = 0; s_cnt_above = 0; s_mabove = 0; }
    for (int d = 3; d >= 0; --d) {
        for (int k = threadIdx.x; k < 256; k += NT) { s_cnt[k] = 0; s_mass[k] = 0; }
        __syncthreads();
        const uint32_t pre = s_prefix;
        const int hi_shift = (d + 1) * 8;
        for (int32_t j = threadIdx.x; j < L; j += NT) {
            const float z = ld_logit<DT>(row, j);
            const uint32_t key = zkey(z);
            if (d < 3 && (key >> hi_shift) != (pre >> hi_shift)) continue;
            const uint32_t dig = (key >> (d * 8)) & 255u;
            const unsigned long long fw = (unsigned long long)((double)exp2_hw((z - m) * c) * kFix);
            atomicAdd(&s_cnt[dig], 1u);
            atomicAdd(&s_mass[dig], fw);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            if (d == 3) {
                unsigned long long tot = 0;
                for (int k = 0; k < 256; ++k) tot += s_mass[k];
                s_total = tot;
                s_T0 = (unsigned long long)((double)top_p * (double)tot);
            }
            unsigned long long above = s_mabove;
            uint32_t cabove = s_cnt_above;
            int sel = -1, lowest = -1;
            for (int k = 255; k >= 0; --k) {
                if (s_cnt[k] == 0) continue;
                lowest = k;
                if (above + s_mass[k] > s_T0) { sel = k; break; }
                above += s_mass[k];
                cabove += s_cnt[k];
            }
            if (sel < 0) {       // rounding left the crossing below every bin: take the last one
                sel = lowest;
                above -= s_mass[sel];
                cabove -= s_cnt[sel];
            }
            s_mabove = above;
            s_cnt_above = cabove;
            s_prefix = pre | ((uint32_t)sel << (d * 8));
            s_g = s_cnt[sel];
        }
        __syncthreads();
    }
    // ties at the boundary key: keep the lowest-id ones while the mass ahead <= T0
    const uint32_t kstar = s_prefix;
    const float zstar = fkey_inv(kstar);
    const unsigned long long fws = (unsigned long long)((double)exp2_hw((zstar - m) * c) * kFix);
    uint32_t tkeep = s_g;
    {
        const unsigned long long room = s_T0 - s_mabove;     // s_mabove <= s_T0 by construction
        if (fws > 0) {
            const unsigned long long q = room / fws + 1;
            if (q < tkeep) tkeep = (uint32_t)q;
        }
    }
    // the tkeep-th tie in id order: contiguous id segments per thread
    const int32_t per = (L + NT - 1) / NT;
    const int32_t j0 = min(L, (int32_t)threadIdx.x * per), j1 = min(L, j0 + per);
    int32_t cnt = 0;
    for (int32_t j = j0; j < j1; ++j) cnt += zkey(ld_logit<DT>(row, j)) == kstar;
    // exclusive scan of counts (as doubles: exact below 2^53)
    __shared__ double s_dtmp[NT / kWave];
    double tot;
    const int32_t before = (int32_t)wg_excl_scan_f64<NT>((double)cnt, s_dtmp, &tot);
    if (threadIdx.x == 0) s_tie_cut = -1;
    __syncthreads();
    if ((uint32_t)before < tkeep && (uint32_t)(before + cnt) >= tkeep) {
        int32_t seen = before;
        for (int32_t j = j0; j < j1; ++j)
            if (zkey(ld_logit<DT>(row, j)) == kstar && ++seen == (int32_t)tkeep) { s_tie_cut = j; break; }
    }
    __syncthreads();
    RowDesc d;
    d.m = m;
    d.Z = (float)((double)s_total / kFix);
    d.Zk = (float)(((double)s_mabove + (double)tkeep * (double)fws) / kFix);
    d.key = kstar;
    d.tie_cut = s_tie_cut;
    d.nkept = (int32_t)(s_cnt_above + tkeep);
    d.flags = RD_FALLBACK;
    d.ptok = 0.0f;
    if (LIST && d.nkept <= kKeptCap) {
        if (threadIdx.x == 0) s_nlist = 0;
        __syncthreads();
        for (int32_t j = threadIdx.x; j < L; j += NT) {
            const float z = ld_logit<DT>(row, j);
            if (row_kept(d, z, j)) {
                const int32_t pos = atomicAdd(&s_nlist, 1);
                if (pos < kKeptCap) {
                    KeptEnt e;
                    e.id = j;
                    e.w = exp2_hw((z - m) * c);
                    pub(&kept[pos], e);
                }
            }
        }
        __syncthreads();
        d.flags |= RD_HAS_LIST;
    }
    if (threadIdx.x == 0) pub(out, d);
}

// ---------------------------------------------------------------------------
// Fixed-point codes and wave helpers of the band selects and list draws.
// ---------------------------------------------------------------------------

// Fixed point for the band select and the list draw: a weight in (0, 1]
// becomes w * 2^48, so up to 65536 units of mass fit a u64 and every sum is
// exact and independent of the order of its terms.
constexpr double kFixSelMaxMass = 60000.0;      // rows with more mass take the exact path

// One step of a wave reduction on a 64-bit value: add the value DPP-moved
// under control CTRL (rows outside ROWMASK add 0).  No LDS traffic.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_add_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWMASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWMASK, 0xf, false);
    return v + (((uint64_t)hi << 32) | lo);
}
// Sum over the 64 lanes, returned to every lane (all lanes must be active):
// pairs, quads, half rows and rows by DPP permutes, then the rows are
// chained through the row broadcasts so that lane 63 holds the total.
__device__ __forceinline__ uint64_t wave_total_u64(uint64_t v) {
    v = dpp_add_u64<0xB1, 0xf>(v);     // quad_perm [1,0,3,2]
    v = dpp_add_u64<0x4E, 0xf>(v);     // quad_perm [2,3,0,1]
    v = dpp_add_u64<0x141, 0xf>(v);    // row_half_mirror
    v = dpp_add_u64<0x140, 0xf>(v);    // row_mirror
    v = dpp_add_u64<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v = dpp_add_u64<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes in lane order (all lanes active):
// shifts by 1, 2, 4, 8 inside each row of 16, then the row totals are carried
// through the row broadcasts.
__device__ __forceinline__ uint64_t wave_incl_scan_u64_dpp(uint64_t v) {
    v = dpp_add_u64<0x111, 0xf>(v);    // row_shr:1
    v = dpp_add_u64<0x112, 0xf>(v);    // row_shr:2
    v = dpp_add_u64<0x114, 0xf>(v);    // row_shr:4
    v = dpp_add_u64<0x118, 0xf>(v);    // row_shr:8
    v = dpp_add_u64<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v = dpp_add_u64<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}

// The same reduction pattern on floats: maximum, then sum, over the wave.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_max_f32(float v) {
    const float w = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROWMASK, 0xf, false));
    return fmaxf(v, w);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add_f32(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, false));
}
// Online-softmax partials (m, s) of the 64 lanes combined, returned to every
// lane: the wave maximum M first, then the sum of s * 2^((m - M) * c).
__device__ __forceinline__ MaxSum wave_maxsum_dpp(MaxSum a, float c) {
    float m = a.m;
    m = dpp_max_f32<0xB1, 0xf>(m);
    m = dpp_max_f32<0x4E, 0xf>(m);
    m = dpp_max_f32<0x141, 0xf>(m);
    m = dpp_max_f32<0x140, 0xf>(m);
    m = dpp_max_f32<0x142, 0xa>(m);
    m = dpp_max_f32<0x143, 0xc>(m);
    MaxSum r;
    r.m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
    float s = a.m > -INFINITY ? a.s * exp2_hw((a.m - r.m) * c) : 0.0f;
    s = dpp_add_f32<0xB1, 0xf>(s);
    s = dpp_add_f32<0x4E, 0xf>(s);
    s = dpp_add_f32<0x141, 0xf>(s);
    s = dpp_add_f32<0x140, 0xf>(s);
    s = dpp_add_f32<0x142, 0xa>(s);
    s = dpp_add_f32<0x143, 0xc>(s);
    r.s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
    return r;
}

// 64-bit values across the lanes of a wave.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
// Lane l takes the value of lane l ^ J, by VALU cross-lane operations (no
// LDS round trip): DPP quad permutes for 1 and 2, two DPP row permutes for 4
// (row half mirror, then quad reverse) and 8 (row mirror, then row half
// mirror), and the permlane swaps for 16 and 32 (with both operands x, lane l
// of an even row or half gets x[l ^ J] in the second result, of an odd one
// in the first).  Every lane of the wave takes part.
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
    if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
    if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
    if constexpr (J == 4) {
        const int t = __builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xf, 0xf, false);
    }
    if constexpr (J == 8) {
        const int t = __builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, t, 0x141, 0xf, 0xf, false);
    }
    if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? r[0] : r[1];
    }
    if constexpr (J == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? r[0] : r[1];
    }
    return v;
}
template <int J>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
    return ((uint64_t)lane_xor_u32<J>((uint32_t)(v >> 32)) << 32) | lane_xor_u32<J>((uint32_t)v);
}
// Lane l takes lane 63 - l: row mirror (l ^ 15), then l ^ 16 and l ^ 32.
__device__ __forceinline__ uint64_t lane_reverse_u64(uint64_t v) {
    auto rev = [](uint32_t x) {
        const uint32_t m = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xf, 0xf, false);
        return lane_xor_u32<32>(lane_xor_u32<16>(m));
    };
    return ((uint64_t)rev((uint32_t)(v >> 32)) << 32) | rev((uint32_t)v);
}

// One compare-exchange stage of a bitonic network over the wave: partner
// l ^ J; the lower lane of the pair keeps the larger when `desc`.
template <int J>
__device__ __forceinline__ uint64_t wave_cx_u64(uint64_t v, bool desc) {
    const uint64_t o = lane_xor_u64<J>(v);
    const bool low = (threadIdx.x & J) == 0;
    return (low == desc) ? (v > o ? v : o) : (v < o ? v : o);
}
// Bitonic sort of one value per lane, descending across the wave (lane 0
// the largest); every lane takes part.  Runs of length k alternate direction
// until the last (k = 64), which is descending.
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t v) {
    const int lane = threadIdx.x & (kWave - 1);
    v = wave_cx_u64<1>(v, (lane & 2) == 0);
    v = wave_cx_u64<2>(v, (lane & 4) == 0);
    v = wave_cx_u64<1>(v, (lane & 4) == 0);
    v = wave_cx_u64<4>(v, (lane & 8) == 0);
    v = wave_cx_u64<2>(v, (lane & 8) == 0);
    v = wave_cx_u64<1>(v, (lane & 8) == 0);
    v = wave_cx_u64<8>(v, (lane & 16) == 0);
    v = wave_cx_u64<4>(v, (lane & 16) == 0);
    v = wave_cx_u64<2>(v, (lane & 16) == 0);
    v = wave_cx_u64<1>(v, (lane & 16) == 0);
    v = wave_cx_u64<16>(v, (lane & 32) == 0);
    v = wave_cx_u64<8>(v, (lane & 32) == 0);
    v = wave_cx_u64<4>(v, (lane & 32) == 0);
    v = wave_cx_u64<2>(v, (lane & 32) == 0);
    v = wave_cx_u64<1>(v, (lane & 32) == 0);
    v = wave_cx_u64<32>(v, true);
    v = wave_cx_u64<16>(v, true);
    v = wave_cx_u64<8>(v, true);
    v = wave_cx_u64<4>(v, true);
    v = wave_cx_u64<2>(v, true);
    v = wave_cx_u64<1>(v, true);
    return v;
}
// The kWave largest of two descending wave lists, descending: the larger of
// a[l] and b[63 - l] in each lane forms a bitonic sequence holding them,
// which a half cleaner network sorts.
__device__ __forceinline__ uint64_t wave_merge_top_u64(uint64_t a, uint64_t b) {
    const uint64_t br = lane_reverse_u64(b);
    uint64_t v = a > br ? a : br;
    v = wave_cx_u64<32>(v, true);
    v = wave_cx_u64<16>(v, true);
    v = wave_cx_u64<8>(v, true);
    v = wave_cx_u64<4>(v, true);
    v = wave_cx_u64<2>(v, true);
    v = wave_cx_u64<1>(v, true);
    return v;
}

// Inclusive prefix sum of a u64 across a wave (lane order).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint64_t w = __shfl_up(v, o, kWave);
        if (lane >= o) v += w;
    }
    return v;
}

// Wave-aggregated LDS append: every lane of the wave calls it; lanes with
// pred get consecutive slots from *counter, with one atomic per wave instead
// of one per lane (same-address LDS atomics serialise lane by lane).
// Inclusive prefix sum of one int per lane over the wave, by DPP row shifts
// and row broadcasts (all lanes active).
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}
// Reserve n slots per lane in a shared list with one LDS atomic per wave;
// returns this lane's first slot.  All lanes call it together.
__device__ __forceinline__ int32_t wave_append_n(int32_t n, int32_t *counter) {
    const int32_t inc = wave_incl_scan_i32(n);
    const int32_t tot = __builtin_amdgcn_readlane(inc, kWave - 1);
    int32_t base = 0;
    if (tot > 0) {
        if ((threadIdx.x & (kWave - 1)) == 0) base = atomicAdd(counter, tot);
        base = __builtin_amdgcn_readlane(base, 0);
    }
    return base + inc - n;
}

__device__ __forceinline__ int32_t wave_append(bool pred, int32_t *counter) {
    const uint64_t bal = __ballot(pred);
    if (bal == 0) return -1;
    const int lane = threadIdx.x & (kWave - 1);
    const int leader = __ffsll((unsigned long long)bal) - 1;
    int32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (int32_t)__popcll(bal));
    base = __builtin_amdgcn_readlane(base, leader);
    return pred ? base + (int32_t)__popcll(bal & ((1ull << lane) - 1ull)) : -1;
}
// Fixed-point weights of band tokens: w in (0, 1] becomes floor(w * 2^31),
// so a u64 holds the exact sum of any band (at most 2048 tokens) and every
// sum is independent of the order of its terms.
constexpr double kFixW = 2147483648.0;          // 2^31
__device__ __forceinline__ uint32_t fixw32(float z, float m, float c) {
    // w * 2^31 is exact in float32 (w <= 1), and the conversion truncates
    return (uint32_t)(exp2_hw((z - m) * c) * 2147483648.0f);
}

// Ordering code of a band token: (key << 32) | ~id.  Token j is ahead of
// token i in the stable order (larger logit first, lower id first among
// equal logits) exactly when P_j > P_i.
__device__ __forceinline__ uint64_t pcode(uint32_t key, int32_t id) {
    return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ uint32_t pkey(uint64_t p) { return (uint32_t)(p >> 32); }
__device__ __forceinline__ int32_t pid(uint64_t p) { return (int32_t)~(uint32_t)p; }

// floor(u * S) exactly, for a float32 u in [0, 1).
__device__ __forceinline__ uint64_t frac_floor(float u, uint64_t S) {
    const uint32_t bits = __float_as_uint(u);
    const uint32_t e = (bits >> 23) & 0xffu;
    const uint64_t m = e ? (uint64_t)((bits & 0x7fffffu) | 0x800000u) : (uint64_t)(bits & 0x7fffffu);
    const int sh = e ? 150 - (int)e : 149;                   // u = m * 2^-sh
    if (sh >= 128) return 0;
    const unsigned __int128 pr = (unsigned __int128)m * S;
    return (uint64_t)(pr >> sh);
}

}  // namespace sv
