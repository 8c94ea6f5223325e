// sv_sample.hip -- sampling verification (speculative sampling).
//
// What is computed ("Ling-3.0-flash-dspark" draft-model tutorial, mlqm.cn,
// sec. 3.1 and the SpeculativeDecoder code of sec. 4.2; SSD inference-engine
// guide, lpnh.cn, sec. 6 for the d2t map):
//   p_i = softmax(top_p(target row i / T)), q_i = softmax(top_p(draft row i / T));
//   draft token x_i is accepted when u_i * q_i(x_i) < p_i(x_i), scanning
//   i = 0.. until the first rejection n; the emitted token after the accepted
//   prefix is drawn with u_s from norm(max(0, p_n - q_n)) when n < gamma, or
//   from p_gamma when every draft was accepted.  Draws are inverse-CDF in
//   ascending token id.
//
// Launch structure (no host synchronization anywhere):
//   top-p on:  one kernel.  One workgroup per row (target and draft rows)
//     streams the row once, keeping the online max / sum-exp per lane and the
//     tokens within a band of the running maximum in LDS; it then sorts that
//     band (bitonic, LDS) by (logit desc, id asc), takes the cumulative mass
//     in that order -- the page's _apply_top_p order -- and writes the kept
//     set (boundary key, tie cut, kept mass, the kept ids and weights).  The
//     last workgroup of each sequence to arrive runs the accept chain and
//     draws from the kept list (a few dozen ids), so the rows are read once.
//     Rows whose band is too crowded, or does not hold top_p of the mass,
//     take an exact radix select over the whole row instead.
//   top-p off: two kernels.  (1) Rows are cut into chunks; each workgroup
//     streams one chunk and writes its (max, sum-exp); the last workgroup of a
//     sequence combines them in chunk order, runs the accept chain and records
//     n.  (2) Tiles of the row to draw from (target row n and draft row n, or
//     the bonus row) are spread over workgroups; each sums its tile's weights;
//     the last one scans the tile sums, finds the tile holding u_s * S and
//     searches inside it.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

// Rarely taken paths (exact whole-row select, wide-band radix, whole-row
// draw).  SV_RARE_OUTLINE keeps them out of line so the common path stays
// compact in the instruction cache; inlined otherwise.
#ifdef SV_RARE_OUTLINE
#define SV_RARE __attribute__((noinline))
#define SV_TOPP_OCCUPANCY __attribute__((amdgpu_waves_per_eu(6)))
#else
#define SV_RARE __forceinline__
#define SV_TOPP_OCCUPANCY
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
__device__ __forceinline__ float wg_sum_f32(float v, float *s_tmp) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = s_tmp[0];
    for (int w = 1; w < NT / kWave; ++w) t += s_tmp[w];
    __syncthreads();
    return t;
}

template <int NT>
__device__ __forceinline__ int32_t wg_sum_i32(int32_t v, int32_t *s_tmp) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = v;
    __syncthreads();
    int32_t t = 0;
    for (int w = 0; w < NT / kWave; ++w) t += s_tmp[w];
    __syncthreads();
    return t;
}

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
// Draw from the residual (or bonus) distribution over target ids [t0, t1):
// weights r_t = max(0, p_n(t) - q_n(t)) when resid, else p_n(t).
// ---------------------------------------------------------------------------
struct DrawCtx {
    const void *trow;          // target row n
    const void *drow;          // draft row n (resid only)
    const int32_t *d2t;
    int32_t Vd;
    RowDesc dp, dq;
    float c;
    bool resid;
};

// Fills s_r[0, t1 - t0) with the weights (and s_q as scratch for d2t).
template <int DTT, int DTD, int NT>
__device__ __forceinline__ void tile_weights(const DrawCtx &x, int32_t t0, int32_t t1, float *s_r, float *s_q) {
    const int32_t len = t1 - t0;
    if (x.resid && x.d2t) {
        for (int32_t k = threadIdx.x; k < len; k += NT) s_q[k] = 0.0f;
        __syncthreads();
        const int32_t j0 = lower_bound_i32(x.d2t, x.Vd, t0);
        const int32_t j1 = lower_bound_i32(x.d2t, x.Vd, t1);
        for (int32_t j = j0 + threadIdx.x; j < j1; j += NT) {
            const int32_t t = x.d2t[j];
            if (t >= t0 && t < t1) s_q[t - t0] = row_prob(x.dq, ld_logit<DTD>(x.drow, j), j, x.c);
        }
        __syncthreads();
    }
    for (int32_t k = threadIdx.x; k < len; k += NT) {
        const int32_t t = t0 + k;
        const float p = row_prob(x.dp, ld_logit<DTT>(x.trow, t), t, x.c);
        float r = p;
        if (x.resid) {
            const float q = x.d2t ? s_q[k] : row_prob(x.dq, ld_logit<DTD>(x.drow, t), t, x.c);
            r = p - q > 0.0f ? p - q : 0.0f;
        }
        s_r[k] = r;
    }
    __syncthreads();
}

// Sum of a tile's weights: per-thread sums in index-stride order, then a
// fixed-order tree.  Deterministic for a given launch shape.
template <int DTT, int DTD, int NT>
__device__ __forceinline__ float tile_mass(const DrawCtx &x, int32_t t0, int32_t t1, float *s_r, float *s_q,
                           float *s_ftmp) {
    tile_weights<DTT, DTD, NT>(x, t0, t1, s_r, s_q);
    float acc = 0.0f;
    for (int32_t k = threadIdx.x; k < t1 - t0; k += NT) acc += s_r[k];
    return wg_sum_f32<NT>(acc, s_ftmp);
}

// Given the tile sums, find the token for u * S; returns -1 when S == 0.
template <int DTT, int DTD, int NT>
__device__ __forceinline__ int32_t draw_from_tiles(const DrawCtx &x, int32_t V, const float *mass, int32_t ntiles,
                                   double u, float *s_r, float *s_q, double *s_dtmp,
                                   int32_t *s_itmp, double *s_bcast) {
    if (threadIdx.x == 0) {
        double S = 0.0;
        auto mt = [&](int32_t t) { return __uint_as_float(sub_u32(&mass[t])); };
        for (int32_t t = 0; t < ntiles; ++t) S += (double)mt(t);
        const double target = u * S;
        double run = 0.0, before = 0.0;
        int32_t tile = -1, lastpos = -1;
        for (int32_t t = 0; t < ntiles; ++t) {
            const float m_t = mt(t);
            if (m_t > 0.0f) lastpos = t;
            before = run;
            run += (double)m_t;
            if (run > target) { tile = t; break; }
        }
        if (tile < 0) { tile = lastpos; before = S - (lastpos >= 0 ? (double)mt(lastpos) : 0.0); }
        s_bcast[0] = S;
        s_bcast[1] = target - before;
        s_bcast[2] = (double)tile;
    }
    __syncthreads();
    const double S = s_bcast[0], tin = s_bcast[1];
    const int32_t tile = (int32_t)s_bcast[2];
    __syncthreads();
    if (!(S > 0.0) || tile < 0) return -1;
    const int32_t t0 = tile * kTile, t1 = min(V, t0 + kTile);
    tile_weights<DTT, DTD, NT>(x, t0, t1, s_r, s_q);
    double tot;
    const int32_t k = wg_inverse_cdf<NT>(t1 - t0, [&](int32_t s) { return s_r[s]; }, tin, false,
                                         s_dtmp, s_itmp, &tot);
    return k < 0 ? -1 : t0 + k;
}

// ---------------------------------------------------------------------------
// The accept chain (shared by both modes); runs in the last workgroup of a
// sequence once every row descriptor of the sequence is in s_rows.
// Returns n and writes p_tok / q_tok / the accepted tokens / padding / len /
// status; the drawn token at position n is written by the caller.
// ---------------------------------------------------------------------------
template <int DTT, int DTD, int NT>
__device__ __forceinline__ int32_t accept_chain(const SampleArgs &a, int32_t b, const RowDesc *s_rows,
                                int32_t *s_itmp, int32_t *s_status) {
    const int32_t g = a.gamma;
    const int32_t *x = a.tokens + (size_t)b * g;
    int32_t first_rej = INT32_MAX;
    for (int32_t i = threadIdx.x; i < g; i += NT) {
        const int32_t t = x[i];
        float pa = 0.0f, qc = 0.0f;
        if (t < 0 || t >= a.Vt) {
            atomicOr(s_status, (int)SV_SEQ_TOKEN_RANGE);
        } else {
            const RowDesc dp = s_rows[i], dq = s_rows[g + 1 + i];
            const void *trow = reinterpret_cast<const char *>(a.tl) +
                               ((size_t)b * (g + 1) + i) * (size_t)a.Vt * Elem<DTT>::kBytes;
            const void *drow = reinterpret_cast<const char *>(a.dl) +
                               ((size_t)b * g + i) * (size_t)a.Vd * Elem<DTD>::kBytes;
            pa = row_prob(dp, ld_logit<DTT>(trow, t), t, a.c);
            if (a.d2t) {
                const int32_t j = lower_bound_i32(a.d2t, a.Vd, t);
                if (j < a.Vd && a.d2t[j] == t) qc = row_prob(dq, ld_logit<DTD>(drow, j), j, a.c);
            } else {
                qc = row_prob(dq, ld_logit<DTD>(drow, t), t, a.c);
            }
        }
        if (a.out_p) a.out_p[(size_t)b * g + i] = pa;
        if (a.out_q) a.out_q[(size_t)b * g + i] = qc;
        // u * q < p, exactly: both products fit a double
        const double u = (double)a.u_acc[(size_t)b * g + i];
        if (!(u * (double)qc < (double)pa) && i < first_rej) first_rej = i;
    }
    const int32_t fr = wg_min_i32<NT>(first_rej, s_itmp);
    const int32_t n = fr == INT32_MAX ? g : fr;
    for (int32_t i = threadIdx.x; i <= g; i += NT)
        if (i != n) a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? x[i] : -1;
    return n;
}

// ---------------------------------------------------------------------------
// Top-p rows: exact radix select over the whole row (fallback path).
// Finds the boundary key by mass with 8-bit digits of the 32-bit key, in
// fixed point (deterministic integer sums), then the tie cut by id, then the
// kept list when it fits.
// ---------------------------------------------------------------------------
constexpr double kFix = 274877906944.0;   // 2^38: w in (0, 1] -> fixed point; 2^24 ids fit in 2^62

template <int DT, int NT>
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
    if (d.nkept <= kKeptCap) {
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
// Top-p kernel: one workgroup per row, then the sequence epilogue.
// ---------------------------------------------------------------------------

// Fixed point for the band select and the list draw: a weight in (0, 1]
// becomes w * 2^48, so up to 65536 units of mass fit a u64 and every sum is
// exact and independent of the order of its terms.
constexpr double kFixSelMaxMass = 60000.0;      // rows with more mass take the exact path

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
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
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint64_t w = __shfl_xor(v, o, kWave);
        v = w < v ? w : v;
    }
    return v;
}

// Fixed-point weights of band tokens: w in (0, 1] becomes floor(w * 2^31),
// so a u64 holds the exact sum of any band (at most 2048 tokens) and every
// sum is independent of the order of its terms.
constexpr double kFixW = 2147483648.0;          // 2^31
__device__ __forceinline__ uint32_t fixw32(float z, float m, float c) {
    return (uint32_t)((double)exp2_hw((z - m) * c) * kFixW);
}

// Ordering code of a band token: (key << 32) | ~id.  Token j is ahead of
// token i in the stable order (larger logit first, lower id first among
// equal logits) exactly when P_j > P_i.
__device__ __forceinline__ uint64_t pcode(uint32_t key, int32_t id) {
    return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ uint32_t pkey(uint64_t p) { return (uint32_t)(p >> 32); }
__device__ __forceinline__ int32_t pid(uint64_t p) { return (int32_t)~(uint32_t)p; }

// Boundary of the kept set by radix select, one wave (lanes 0..63), for
// bands too wide for the pairwise test.  The boundary key is the largest
// key K with M(>K) <= T0 < M(>=K) (M = band mass of the keys above K),
// found digit by digit (8-bit digits of the key, most significant first)
// from LDS histograms of count and fixed-point mass, scanning bins from the
// top.  Of the g tokens on it, the lowest-id min(g, floor((T0 - M(>K)) / w)
// + 1) are kept.  Writes the boundary key / tie cut / kept count / kept mass
// to the four result slots.
__device__ SV_RARE void band_radix(const uint64_t *s_P, const uint32_t *s_fw, unsigned char *s_bins,
                                           int32_t n, uint64_t T0f, uint32_t *r_key, int32_t *r_tc,
                                           int32_t *r_nk, uint64_t *r_zk) {
    const int lane = threadIdx.x;
    uint32_t *bcnt = reinterpret_cast<uint32_t *>(s_bins);                  // [256]
    uint64_t *bmass = reinterpret_cast<uint64_t *>(s_bins + 1024);          // [256]
    uint32_t prefix = 0;
    uint64_t above = 0;
    int32_t cab = 0, g = 0;
    for (int d = 3; d >= 0; --d) {
        const int sh = 8 * d;
#pragma unroll
        for (int q = 0; q < 4; ++q) { bcnt[lane * 4 + q] = 0; bmass[lane * 4 + q] = 0; }
        __builtin_amdgcn_wave_barrier();
        for (int32_t i = lane; i < n; i += kWave) {
            const uint32_t k = pkey(s_P[i]);
            if (d < 3 && (k >> (sh + 8)) != (prefix >> (sh + 8))) continue;
            const uint32_t dig = (k >> sh) & 255u;
            atomicAdd(&bcnt[dig], 1u);
            atomicAdd(reinterpret_cast<unsigned long long *>(&bmass[dig]), (unsigned long long)s_fw[i]);
        }
        __builtin_amdgcn_wave_barrier();
        // lane l owns bins 255-4l .. 252-4l, so lane order is descending bin order
        uint64_t bm[4];
        uint32_t bc[4];
        uint64_t m4 = 0;
        uint32_t c4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bm[q] = bmass[255 - 4 * lane - q];
            bc[q] = bcnt[255 - 4 * lane - q];
            m4 += bm[q];
            c4 += bc[q];
        }
        const uint64_t incl = wave_incl_scan_u64(m4);
        const int32_t cincl = (int32_t)wave_incl_scan_u64((uint64_t)c4);
        uint64_t run = above + incl - m4;              // mass of the bins above this lane's
        int32_t crun = cab + cincl - (int32_t)c4;
        int sel = -1, lowest = -1, lq = 0;
        uint64_t sel_above = 0;
        int32_t sel_cab = 0;
        uint32_t sel_g = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (sel < 0 && bc[q] > 0 && run + bm[q] > T0f) {
                sel = 255 - 4 * lane - q;
                sel_above = run;
                sel_cab = crun;
                sel_g = bc[q];
            }
            if (bc[q] > 0) { lowest = 255 - 4 * lane - q; lq = q; }
            run += bm[q];
            crun += (int32_t)bc[q];
        }
        const uint64_t hasb = __ballot(sel >= 0);
        int src;
        if (hasb) {
            src = __ffsll((unsigned long long)hasb) - 1;
        } else {
            // rounding left the crossing below every bin: take the lowest non-empty one
            if (lowest >= 0) {
                sel = lowest;
                uint64_t r2 = above + incl - m4;
                int32_t c2 = cab + cincl - (int32_t)c4;
                for (int q = 0; q < lq; ++q) { r2 += bm[q]; c2 += (int32_t)bc[q]; }
                sel_above = r2;
                sel_cab = c2;
                sel_g = bc[lq];
            }
            src = 63 - __clzll((unsigned long long)__ballot(lowest >= 0));
        }
        const int dig = __shfl(sel, src, kWave);
        above = __shfl(sel_above, src, kWave);
        cab = __shfl(sel_cab, src, kWave);
        g = (int32_t)__shfl(sel_g, src, kWave);
        prefix |= (uint32_t)dig << sh;
        __builtin_amdgcn_wave_barrier();
    }
    const uint32_t ks = prefix;
    // every boundary tie has the same fixed-point weight
    uint32_t wsv = 0;
    for (int32_t i = lane; i < n; i += kWave)
        if (pkey(s_P[i]) == ks) wsv = s_fw[i];
    const uint64_t ws = (uint64_t)wave_max(wsv);
    int32_t tkeep = g;
    if (ws > 0 && above <= T0f) {
        const uint64_t q = (T0f - above) / ws + 1;
        if (q < (uint64_t)tkeep) tkeep = (int32_t)q;
    }
    // the tkeep-th boundary tie in id order: the tie whose count of ties
    // with a lower id is tkeep - 1
    int32_t tc = -1;
    for (int32_t i = lane; i < n; i += kWave) {
        if (pkey(s_P[i]) != ks) continue;
        const int32_t id = pid(s_P[i]);
        int32_t rank = 0;
        for (int32_t j = 0; j < n; ++j) rank += (pkey(s_P[j]) == ks && pid(s_P[j]) < id) ? 1 : 0;
        if (rank == tkeep - 1) tc = id;
    }
    tc = wave_max(tc);
    if (lane == 0) {
        *r_key = ks;
        *r_tc = tc;
        *r_nk = cab + tkeep;
        *r_zk = above + (uint64_t)tkeep * ws;
    }
}

// One top-p row: stream it once (online max / sum-exp per lane; 16-byte
// vectors whose maximum is within the band of the running row maximum are
// copied to LDS), then expand the band, select the kept set, and publish the
// row descriptor and kept list.  s_lds is 32 KiB: band tokens in its first
// half, band vectors in its second.
template <int DT, int NT, int U>
__device__ __forceinline__ void topp_row(const void *row, int32_t L, float c, float band, float top_p, RowDesc *out,
                                         KeptEnt *kept, uint64_t *s_lds, int32_t *s_cvid, int32_t xtok,
                                         const int32_t *d2t) {
    __shared__ uint32_t s_maxkey;
    __shared__ int32_t s_ncand, s_nvec, s_nsel, s_nk, s_nlist;
    __shared__ float s_mred[NT / kWave], s_sred[NT / kWave];
    __shared__ unsigned long long s_bmass[4], s_zk, s_pmin;
    __shared__ float s_ptok;
    uint64_t *s_cand = s_lds;                                          // [kCandCap] band tokens
    u32x4 *s_cvec = reinterpret_cast<u32x4 *>(s_lds + kCandCap);       // [kCandVecCap] band vectors
    uint64_t *s_P = s_lds + kCandCap;                                  // [kCandCap] after expansion
    uint32_t *s_fw = reinterpret_cast<uint32_t *>(s_lds + 2 * kCandCap);            // [kCandCap]
    uint64_t *s_ahead = s_lds + 2 * kCandCap + kCandCap / 2;                        // [NT] / radix bins

    if (threadIdx.x == 0) { s_maxkey = fkey(-INFINITY); s_ncand = 0; s_nvec = 0; s_nlist = 0; }
    __syncthreads();

    using E = Elem<DT>;
    float m_l = -INFINITY, s_l = 0.0f;
    const RowSplit sp = row_split<DT>(row, L);
    auto scalar_elem = [&](float z) {
        if (z > m_l) { s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - z) * c); m_l = z; }
        s_l += exp2_hw((z - m_l) * c);
        if (z > -INFINITY) atomicMax(&s_maxkey, zkey(z));
    };
    if (threadIdx.x < sp.head) scalar_elem(E::load(row, threadIdx.x));
    const u32x4 *body = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(row) +
                                                        (size_t)sp.head * E::kBytes);
    // One iteration's U vectors per lane.  The running row maximum is shared
    // through LDS: a lane publishes (atomicMax on the key) only when its tile
    // maximum beats the shared value it read, rare after the first iteration.
    auto tile = [&](const u32x4 (&raw)[U], const float (&xv)[U][E::kPerVec], const float (&vm)[U], float tm,
                    int32_t vbase, int nu) {
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - tm) * c);
            m_l = tm;
        }
        const float mc = m_l * c;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < nu) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) s_l += exp2_hw(fmaf(xv[u][k], c, -mc));
            }
        float smax = fkey_inv(s_maxkey);
        if (tm > smax) {
            atomicMax(&s_maxkey, zkey(tm));
            smax = tm;
        }
        const float thr = smax - band;
        // band vectors are rare (a fraction of a percent): one LDS atomic each
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < nu && vm[u] >= thr) {
                const int32_t pos = atomicAdd(&s_nvec, 1);
                if (pos < kCandVecCap) {
                    s_cvec[pos] = raw[u];
                    s_cvid[pos] = vbase + u * NT;
                }
            }
    };
    auto load_iter = [&](int32_t it, u32x4 (&raw)[U], float (&xv)[U][E::kPerVec], float (&vm)[U],
                         float &tm) -> int {
        const int32_t vbase = it * U * NT + threadIdx.x;
        int nu = 0;
        tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vm[u] = -INFINITY;
            if (vbase + u * NT < sp.nvec) {
                raw[u] = __builtin_nontemporal_load(&body[vbase + u * NT]);
                E::unpack(raw[u], xv[u]);
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) vm[u] = fmaxf(vm[u], xv[u][k]);
                tm = fmaxf(tm, vm[u]);
                nu = u + 1;
            }
        }
        return nu;
    };
    const int32_t full = sp.nvec / (U * NT);
    const int32_t iters = (sp.nvec + U * NT - 1) / (U * NT);
    if (iters > 0) {
        // iteration 0: take the workgroup-wide maximum first, so the band
        // starts near the row maximum instead of each lane's own tile maximum
        u32x4 raw[U];
        float xv[U][E::kPerVec], vm[U], tm;
        const int nu = load_iter(0, raw, xv, vm, tm);
        const float wm = wave_max(tm);
        if ((threadIdx.x & (kWave - 1)) == 0 && wm > -INFINITY) atomicMax(&s_maxkey, zkey(wm));
        __syncthreads();
        tile(raw, xv, vm, tm, threadIdx.x, nu);
    }
    for (int32_t it = 1; it < full; ++it) {
        const int32_t vbase = it * U * NT + threadIdx.x;
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[vbase + u * NT]);
        float xv[U][E::kPerVec], vm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            E::unpack(raw[u], xv[u]);
            vm[u] = xv[u][0];
#pragma unroll
            for (int k = 1; k < E::kPerVec; ++k) vm[u] = fmaxf(vm[u], xv[u][k]);
        }
        float tm = vm[0];
#pragma unroll
        for (int u = 1; u < U; ++u) tm = fmaxf(tm, vm[u]);
        tile(raw, xv, vm, tm, vbase, U);
    }
    if (iters > full && full > 0) {
        u32x4 raw[U];
        float xv[U][E::kPerVec], vm[U], tm;
        const int nu = load_iter(full, raw, xv, vm, tm);
        tile(raw, xv, vm, tm, full * U * NT + threadIdx.x, nu);
    }
    if (threadIdx.x < sp.tail) scalar_elem(E::load(row, sp.head + sp.nvec * E::kPerVec + threadIdx.x));
    // What follows is short and on the critical path, while other workgroups
    // on this CU are still streaming: issue ahead of their waves.
    __builtin_amdgcn_s_setprio(3);

    // ---- row max and mass ----
    MaxSum ms;
    ms.m = m_l;
    ms.s = s_l;
    ms = wave_maxsum(ms, c);
    if ((threadIdx.x & (kWave - 1)) == 0) { s_mred[threadIdx.x / kWave] = ms.m; s_sred[threadIdx.x / kWave] = ms.s; }
    __syncthreads();
    MaxSum tot;
    tot.m = s_mred[0];
    tot.s = s_sred[0];
    for (int w = 1; w < NT / kWave; ++w) {
        MaxSum o;
        o.m = s_mred[w];
        o.s = s_sred[w];
        tot = maxsum_merge(tot, o, c);
    }
    const float m = tot.m, Z = tot.s;
    if (bad_max(m)) {
        if (threadIdx.x == 0) {
            RowDesc d;
            d.m = m; d.Z = 0.0f; d.Zk = 0.0f; d.key = 0xffffffffu; d.tie_cut = -1;
            d.nkept = 0; d.flags = RD_NO_MASS | RD_HAS_LIST; d.ptok = 0.0f;
            pub(out, d);
        }
        return;
    }

    // ---- expand the band: every token with z >= m - band ----
    const float thr_final = m - band;
    const int32_t nvc = s_nvec;
    bool fallback = nvc > kCandVecCap;
    if (!fallback) {
        // called by every lane of every wave (wave-aggregated append)
        auto put = [&](bool valid, float z, int32_t j) {
            const bool in = valid && z >= thr_final && z > -INFINITY;
            const int32_t pos = wave_append(in, &s_ncand);
            if (in && pos < kCandCap) s_cand[pos] = ((uint64_t)zkey(z) << 32) | (uint32_t)j;
        };
        for (int32_t t0 = 0; t0 < nvc; t0 += NT) {
            const int32_t t = t0 + (int32_t)threadIdx.x;
            const bool valid = t < nvc;
            float x[E::kPerVec];
            int32_t i0 = 0;
            if (valid) {
                E::unpack(s_cvec[t], x);
                i0 = sp.head + s_cvid[t] * E::kPerVec;
            } else {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) x[k] = -INFINITY;
            }
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) put(valid, x[k], i0 + k);
        }
        {
            const bool vh = threadIdx.x < (unsigned)sp.head;
            put(vh, vh ? E::load(row, threadIdx.x) : -INFINITY, threadIdx.x);
            const int32_t jt = sp.head + sp.nvec * E::kPerVec + threadIdx.x;
            const bool vt = threadIdx.x < (unsigned)sp.tail;
            put(vt, vt ? E::load(row, jt) : -INFINITY, jt);
        }
        if (threadIdx.x < 4) s_bmass[threadIdx.x] = 0;
        if (threadIdx.x == 0) { s_nsel = 0; s_nk = 0; s_zk = 0; s_pmin = ~0ull; s_ptok = 0.0f; }
        __syncthreads();
        const int32_t nc = s_ncand;
        const double T0 = (double)top_p * (double)Z;
        fallback = nc > kCandCap || !(T0 < kFixSelMaxMass);
        if (!fallback) {
            const uint64_t T0f = (uint64_t)(T0 * kFixW);
            // sub-bands of 4, 5, 6 and the full band: the smallest one holding
            // more than T0 contains the boundary and every token ahead of it
            const float w4 = 4.0f * (band / kToppBandNats), w5 = 5.0f * (band / kToppBandNats),
                        w6 = 6.0f * (band / kToppBandNats);
            auto subband = [&](float z) { const float dz = m - z; return dz <= w4 ? 0 : dz <= w5 ? 1 : dz <= w6 ? 2 : 3; };
            for (int32_t i = threadIdx.x; i < nc; i += NT) {
                const float z = fkey_inv((uint32_t)(s_cand[i] >> 32));
                atomicAdd(reinterpret_cast<unsigned long long *>(&s_bmass[subband(z)]),
                          (unsigned long long)fixw32(z, m, c));
            }
            __syncthreads();
            int sb = -1;
            {
                uint64_t acc = 0;
                for (int q = 0; q < 4 && sb < 0; ++q) {
                    acc += s_bmass[q];
                    if ((double)acc > (double)T0f * (1.0 + 1e-5)) sb = q;
                }
            }
            fallback = sb < 0;
            if (!fallback) {
                for (int32_t i0 = 0; i0 < nc; i0 += NT) {
                    const int32_t i = i0 + (int32_t)threadIdx.x;
                    uint32_t k = 0;
                    float z = -INFINITY;
                    if (i < nc) {
                        k = (uint32_t)(s_cand[i] >> 32);
                        z = fkey_inv(k);
                    }
                    const bool in = i < nc && subband(z) <= sb;
                    const int32_t pos = wave_append(in, &s_nsel);
                    if (in) {
                        s_P[pos] = pcode(k, (int32_t)(uint32_t)s_cand[i]);
                        s_fw[pos] = fixw32(z, m, c);
                    }
                }
                __syncthreads();
                const int32_t n2 = s_nsel;
                if (n2 <= NT) {
                    // pairwise: token i is kept iff the mass strictly ahead of
                    // it is <= T0.  Each token sums (count << 48 | mass) over
                    // the tokens ahead of it (S slices of the j range per
                    // token); the last kept token is the one with
                    // ahead <= T0 < ahead + w (the band mass exceeds T0, so it
                    // exists and is unique): it records the boundary, the kept
                    // count and the kept mass.
                    const int32_t S = NT / n2;
                    const int t = threadIdx.x;
                    if (S > 1)
                        for (int32_t k = t; k < n2; k += NT) s_ahead[k] = 0;
                    __syncthreads();
                    uint64_t acc = 0;
                    if (t < n2 * S) {
                        const int32_t i = t % n2, sl = t / n2;
                        const int32_t j0 = (int32_t)((int64_t)n2 * sl / S), j1 = (int32_t)((int64_t)n2 * (sl + 1) / S);
                        const uint64_t Pi = s_P[i];
                        for (int32_t j = j0; j < j1; ++j)
                            acc += s_P[j] > Pi ? ((1ull << 48) | (uint64_t)s_fw[j]) : 0ull;
                        if (S > 1) atomicAdd(reinterpret_cast<unsigned long long *>(&s_ahead[i]), (unsigned long long)acc);
                    }
                    if (S > 1) {
                        __syncthreads();
                        if (t < n2) acc = s_ahead[t];
                    }
                    if (t < n2) {
                        const uint64_t ahead = acc & ((1ull << 48) - 1ull);
                        const uint64_t w = s_fw[t];
                        if (ahead <= T0f && ahead + w > T0f) {
                            s_pmin = s_P[t];
                            s_zk = ahead + w;
                            s_nk = (int32_t)(acc >> 48) + 1;
                        }
                    }
                    __syncthreads();
                } else {
                    if (threadIdx.x < kWave) {
                        uint32_t ks;
                        int32_t tc, nk;
                        uint64_t zk;
                        band_radix(s_P, s_fw, reinterpret_cast<unsigned char *>(s_ahead), n2, T0f, &ks, &tc, &nk, &zk);
                        if (threadIdx.x == 0) { s_pmin = pcode(ks, tc); s_nk = nk; s_zk = zk; }
                    }
                    __syncthreads();
                }
                // publish: the kept list (order free), the token's probability,
                // and the row descriptor
                const uint64_t pmin = s_pmin;
                const float Zk = (float)((double)s_zk / kFixW);
                const int32_t nsel = s_nsel;
                for (int32_t i0 = 0; i0 < nsel; i0 += NT) {
                    const int32_t i = i0 + (int32_t)threadIdx.x;
                    const uint64_t P = i < nsel ? s_P[i] : 0ull;
                    const bool in = i < nsel && P >= pmin;
                    const int32_t pos = wave_append(in, &s_nlist);
                    if (in) {
                        const int32_t id = pid(P);
                        KeptEnt e;
                        e.id = id;
                        e.w = exp2_hw((fkey_inv(pkey(P)) - m) * c);
                        pub(&kept[pos], e);
                        if (xtok >= 0 && (d2t ? d2t[id] == xtok : id == xtok)) s_ptok = e.w / Zk;
                    }
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    RowDesc d;
                    d.m = m;
                    d.Z = Z;
                    d.Zk = Zk;
                    d.key = pkey(pmin);
                    d.tie_cut = pid(pmin);
                    d.nkept = s_nk;
                    d.flags = RD_HAS_LIST;
                    d.ptok = s_ptok;
                    pub(out, d);
                }
            }
        }
    }
    if (fallback) {
        topp_exact_row<DT, NT>(row, L, m, c, top_p, out, kept, reinterpret_cast<unsigned char *>(s_lds));
        // the token's probability from the descriptor and its logit
        if (threadIdx.x == 0) {
            RowDesc d = sub(out);
            float pt = 0.0f;
            if (xtok >= 0) {
                int32_t j = xtok;
                if (d2t) {
                    j = lower_bound_i32(d2t, L, xtok);
                    if (j >= L || d2t[j] != xtok) j = -1;
                }
                if (j >= 0 && j < L) pt = row_prob(d, E::load(row, j), j, c);
            }
            d.ptok = pt;
            pub(out, d);
        }
    }
}

// List-based draw for top-p rows: the kept ids of target row n with their
// weights, minus q_n at those ids when drawing a replacement (the residual
// vanishes outside p's kept set).  q_n comes from the draft row's own kept
// list (its ids mapped through d2t when present) when it has one, else from
// its logits.  With K <= NT entries each thread owns one and sums, in fixed
// point, the weights of every entry with an id <= its own: the inclusive CDF
// in id order without sorting, exact and deterministic.  Larger lists are
// sorted by id in LDS first.  s_lds is at least 40 KiB.
template <int DTT, int DTD, int NT>
__device__ __forceinline__ int32_t draw_from_list(const SampleArgs &a, int32_t b, int32_t n, const RowDesc &dp,
                                                  const RowDesc &dq, const KeptEnt *list, const KeptEnt *qlist,
                                                  uint64_t *s_lds, double u, double *s_dtmp, int32_t *s_itmp) {
    const int32_t g = a.gamma;
    const int32_t K = dp.nkept;
    const bool resid = n < g;
    const void *drow = resid ? reinterpret_cast<const char *>(a.dl) +
                                   ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                             : nullptr;
    // q's kept list in LDS as (target id, q) pairs
    const int32_t Kq = (resid && (dq.flags & RD_HAS_LIST) && dq.nkept <= kQListCap) ? dq.nkept : -1;
    int32_t *s_qid = reinterpret_cast<int32_t *>(s_lds);                     // [kQListCap]
    float *s_qv = reinterpret_cast<float *>(s_lds) + kQListCap;              // [kQListCap]
    uint64_t *s_work = s_lds + kQListCap;                                    // past the q list
    // one round trip for both lists: this thread's p entry and q entries
    KeptEnt e;
    e.id = INT32_MAX;
    e.w = 0.0f;
    if (K <= NT && (int32_t)threadIdx.x < K) e = sub(&list[threadIdx.x]);
    for (int32_t j = threadIdx.x; j < Kq; j += NT) {
        const KeptEnt qe = sub(&qlist[j]);
        s_qid[j] = a.d2t ? a.d2t[qe.id] : qe.id;
        s_qv[j] = qe.w / dq.Zk;
    }
    __syncthreads();
    auto weight = [&](const KeptEnt &pe, bool use_resid) -> float {
        float r = pe.w / dp.Zk;
        if (use_resid) {
            float q = 0.0f;
            if (Kq >= 0) {
                for (int32_t j = 0; j < Kq; ++j)
                    if (s_qid[j] == pe.id) q = s_qv[j];
            } else if (a.d2t) {
                const int32_t j = lower_bound_i32(a.d2t, a.Vd, pe.id);
                if (j < a.Vd && a.d2t[j] == pe.id) q = row_prob(dq, ld_logit<DTD>(drow, j), j, a.c);
            } else {
                q = row_prob(dq, ld_logit<DTD>(drow, pe.id), pe.id, a.c);
            }
            r = r - q > 0.0f ? r - q : 0.0f;
        }
        return r;
    };
    if (K <= NT) {
        int32_t *s_id = reinterpret_cast<int32_t *>(s_work);                 // [NT]
        uint64_t *s_rf = s_work + NT / 2;                                    // [NT]
        int32_t *s_tok = reinterpret_cast<int32_t *>(s_work + NT / 2 + NT);  // [1]
        for (int attempt = 0; attempt < 2; ++attempt) {
            const bool use_resid = resid && attempt == 0;
            uint64_t rf = 0;
            if ((int32_t)threadIdx.x < K) {
                rf = (uint64_t)((double)weight(e, use_resid) * kFixW);
                s_id[threadIdx.x] = e.id;
                s_rf[threadIdx.x] = rf;
            }
            if (threadIdx.x == 0) *s_tok = -1;
            __syncthreads();
            uint64_t incl = 0, S = 0;
            for (int32_t j = 0; j < K; ++j) {
                const uint64_t r = s_rf[j];
                S += r;
                if (s_id[j] <= e.id) incl += r;
            }
            if (S > 0) {
                // exactly one entry (in id order) brackets the target
                const uint64_t target = (uint64_t)(u * (double)S);
                if ((int32_t)threadIdx.x < K && rf > 0 && incl > target && incl - rf <= target) *s_tok = e.id;
                __syncthreads();
                return *s_tok;
            }
            if (!use_resid) return -1;
            // zero residual mass (only with p == q on p's support): draw from p_n
            __syncthreads();
        }
        return -1;
    }
    const int P = pow2_at_least(K < 2 ? 2 : K);
    for (int attempt = 0; attempt < 2; ++attempt) {
        const bool use_resid = resid && attempt == 0;
        __syncthreads();
        for (int32_t s = threadIdx.x; s < P; s += NT) {
            uint64_t v = ~0ull;
            if (s < K) {
                const KeptEnt e = sub(&list[s]);
                v = ((uint64_t)(uint32_t)e.id << 32) | __float_as_uint(weight(e, use_resid));
            }
            s_work[s] = v;
        }
        bitonic_sort_u64<NT>(s_work, P);
        double S;
        const int32_t k = wg_inverse_cdf<NT>(
            K, [&](int32_t s) { return __uint_as_float((uint32_t)s_work[s]); }, u, true, s_dtmp, s_itmp, &S);
        if (S > 0.0) return k < 0 ? -1 : (int32_t)(s_work[k] >> 32);
        if (!use_resid) return -1;
    }
    return -1;
}

// Draw over the whole target row n tile by tile (top-p rows whose kept set
// is too large for a list); one workgroup, out of line (rarely taken).
template <int DTT, int DTD, int NT>
__device__ SV_RARE int32_t draw_full_row(const SampleArgs &a, int32_t b, int32_t n, RowDesc dp,
                                                           RowDesc dq, double u, float *s_r, double *s_dtmp,
                                                           int32_t *s_itmp, double *s_bcast) {
    const int32_t g = a.gamma;
    DrawCtx x;
    x.trow = reinterpret_cast<const char *>(a.tl) + ((size_t)b * (g + 1) + n) * (size_t)a.Vt * Elem<DTT>::kBytes;
    x.drow = n < g ? reinterpret_cast<const char *>(a.dl) + ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                   : nullptr;
    x.d2t = a.d2t;
    x.Vd = a.Vd;
    x.dp = dp;
    x.dq = dq;
    x.c = a.c;
    float *s_q = s_r + kTile;
    float *mass = a.tile_mass + (size_t)b * a.ntiles;
    int32_t tok = -1;
    for (int attempt = 0; attempt < 2 && tok < 0; ++attempt) {
        x.resid = n < g && attempt == 0;
        if (attempt == 1 && !(n < g)) break;
        for (int32_t t = 0; t < a.ntiles; ++t) {
            const float mt = tile_mass<DTT, DTD, NT>(x, t * kTile, min(a.Vt, (t + 1) * kTile), s_r, s_q,
                                                     reinterpret_cast<float *>(s_dtmp));
            if (threadIdx.x == 0) pub_u32(&mass[t], __float_as_uint(mt));
        }
        __syncthreads();
        tok = draw_from_tiles<DTT, DTD, NT>(x, a.Vt, mass, a.ntiles, u, s_r, s_q, s_dtmp, s_itmp, s_bcast);
    }
    return tok;
}

// With the rare paths out of line, three 512-thread workgroups per CU (24
// waves, <= 80 VGPRs) keep every row of a 64 x 11-row batch resident.
template <int DTT, int DTD, int NT, int U>
__global__ __launch_bounds__(NT) SV_TOPP_OCCUPANCY void topp_kernel(SampleArgs a) {
    // 44 KiB: band tokens | band vectors, then ordering codes | fixed-point
    // weights | pairwise sums or radix bins; the epilogue reuses it
    __shared__ uint64_t s_cand[2 * kCandCap + kCandCap / 2 + 512];
    __shared__ int32_t s_cvid[kCandVecCap];
    static_assert(sizeof(uint64_t) * kCandCap == 16 * kCandVecCap, "band vectors fill the second quarter");
    static_assert(512 * sizeof(uint64_t) >= 3072 && NT <= 512, "pairwise sums / radix bins / tie ids");
    static_assert(sizeof(RowDesc) * (2 * SV_MAX_GAMMA + 1) <= sizeof(uint64_t) * 4096,
                  "row descriptors must fit the band area");
    static_assert(sizeof(uint64_t) * kKeptCap <= sizeof(uint64_t) * 4096, "list sort must fit the band area");
    static_assert(2 * kTile * sizeof(float) <= sizeof(uint64_t) * 4096, "draw tiles must fit the band area");
    __shared__ int last_flag;
    __shared__ int32_t s_itmp[NT / kWave];
    __shared__ double s_dtmp[NT / kWave];
    __shared__ int32_t s_status;
    __shared__ double s_bcast[4];

    const int32_t g = a.gamma, NR = 2 * g + 1;
    const int32_t b = blockIdx.x / NR, r = blockIdx.x % NR;
    const float band = kToppBandNats * a.T;
    RowDesc *rows = a.rows + (size_t)b * NR;
    KeptEnt *kept = a.kept + ((size_t)b * NR + r) * kKeptCap;
    {
        // row r: target rows 0..g, then draft rows; each carries the draft
        // token it scores (none for the bonus row)
        const bool tgt = r <= g;
        const void *row = tgt ? reinterpret_cast<const void *>(reinterpret_cast<const char *>(a.tl) +
                                                               ((size_t)b * (g + 1) + r) * (size_t)a.Vt * Elem<DTT>::kBytes)
                              : reinterpret_cast<const void *>(reinterpret_cast<const char *>(a.dl) +
                                                               ((size_t)b * g + (r - g - 1)) * (size_t)a.Vd * Elem<DTD>::kBytes);
        const int32_t xt = tgt ? (r < g ? a.tokens[(size_t)b * g + r] : -1) : a.tokens[(size_t)b * g + (r - g - 1)];
        const int32_t *map = tgt ? nullptr : a.d2t;
        if constexpr (DTT == DTD) {
            topp_row<DTT, NT, U>(row, tgt ? a.Vt : a.Vd, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
        } else {
            if (tgt)
                topp_row<DTT, NT, U>(row, a.Vt, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
            else
                topp_row<DTD, NT, U>(row, a.Vd, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
        }
    }

    if (!arrive_last(&a.cnt_stats[b], (uint32_t)NR, &last_flag)) return;

    // ---- sequence epilogue: accept chain, then the draw ----
    RowDesc *s_rows = reinterpret_cast<RowDesc *>(s_cand);   // the row work is done
    for (int32_t k = threadIdx.x; k < NR; k += NT) s_rows[k] = sub(&rows[k]);
    if (threadIdx.x == 0) s_status = 0;
    __syncthreads();
    for (int32_t k = threadIdx.x; k < NR; k += NT)
        if (s_rows[k].flags & RD_NO_MASS) atomicOr(&s_status, (int)SV_SEQ_NO_MASS);
    int32_t n;
    {
        // every row has published the probability of its own draft token
        const int32_t *x = a.tokens + (size_t)b * g;
        int32_t first_rej = INT32_MAX;
        for (int32_t i = threadIdx.x; i < g; i += NT) {
            const int32_t t = x[i];
            if (t < 0 || t >= a.Vt) atomicOr(&s_status, (int)SV_SEQ_TOKEN_RANGE);
            const float pa = s_rows[i].ptok, qc = s_rows[g + 1 + i].ptok;
            if (a.out_p) a.out_p[(size_t)b * g + i] = pa;
            if (a.out_q) a.out_q[(size_t)b * g + i] = qc;
            const double uu = (double)a.u_acc[(size_t)b * g + i];
            if (!(uu * (double)qc < (double)pa) && i < first_rej) first_rej = i;
        }
        const int32_t fr = wg_min_i32<NT>(first_rej, s_itmp);
        n = fr == INT32_MAX ? g : fr;
        for (int32_t i = threadIdx.x; i <= g; i += NT)
            if (i != n) a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? x[i] : -1;
    }
    const RowDesc dp = s_rows[n];
    const RowDesc dq = n < g ? s_rows[g + 1 + n] : dp;
    const double u = (double)a.u_s[b];
    __syncthreads();                                          // s_rows is reused below
    int32_t tok;
    if (dp.flags & RD_HAS_LIST) {
        tok = draw_from_list<DTT, DTD, NT>(a, b, n, dp, dq, a.kept + ((size_t)b * NR + n) * kKeptCap,
                                           a.kept + ((size_t)b * NR + g + 1 + n) * kKeptCap, s_cand, u,
                                           s_dtmp, s_itmp);
    } else {
        // kept set too large for a list: tile-by-tile over the whole row
        tok = draw_full_row<DTT, DTD, NT>(a, b, n, dp, dq, u, reinterpret_cast<float *>(s_cand), s_dtmp, s_itmp,
                                          s_bcast);
    }
    if (threadIdx.x == 0) {
        a.out_tokens[(size_t)b * (g + 1) + n] = tok;
        a.out_len[b] = n;
        if (a.out_status) a.out_status[b] = s_status;
    }
}

// ---------------------------------------------------------------------------
// Plain mode (no top-p): chunked statistics + chain, then the tiled draw.
// ---------------------------------------------------------------------------
template <int DT, int NT, int U>
__device__ __forceinline__ MaxSum chunk_maxsum(const void *row, int32_t L, int32_t chunk, int32_t C, float c,
                               float *s_m, float *s_s) {
    const RowSplit sp = row_split<DT>(row, L);
    const int32_t lo = (int32_t)(((int64_t)sp.nvec * chunk) / C);
    const int32_t hi = (int32_t)(((int64_t)sp.nvec * (chunk + 1)) / C);
    using E = Elem<DT>;
    float m_l = -INFINITY, s_l = 0.0f;
    auto one = [&](float z) {
        if (z > m_l) { s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - z) * c); m_l = z; }
        s_l += exp2_hw((z - m_l) * c);
    };
    if (chunk == 0 && threadIdx.x < sp.head) one(E::load(row, threadIdx.x));
    const u32x4 *body = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(row) +
                                                        (size_t)sp.head * E::kBytes);
    int32_t v = lo + threadIdx.x;
    for (; v + (U - 1) * NT < hi; v += U * NT) {
        float xv[U][E::kPerVec];
#pragma unroll
        for (int u = 0; u < U; ++u) E::unpack(__builtin_nontemporal_load(&body[v + u * NT]), xv[u]);
        float tm = xv[0][0];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) tm = fmaxf(tm, xv[u][k]);
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - tm) * c);
            m_l = tm;
        }
        const float mc = m_l * c;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) s_l += exp2_hw(fmaf(xv[u][k], c, -mc));
    }
    for (; v < hi; v += NT) {
        float xv[E::kPerVec];
        E::unpack(__builtin_nontemporal_load(&body[v]), xv);
#pragma unroll
        for (int k = 0; k < E::kPerVec; ++k) one(xv[k]);
    }
    if (chunk == C - 1 && threadIdx.x < sp.tail) one(E::load(row, sp.head + sp.nvec * E::kPerVec + threadIdx.x));
    MaxSum ms;
    ms.m = m_l;
    ms.s = s_l;
    ms = wave_maxsum(ms, c);
    if ((threadIdx.x & (kWave - 1)) == 0) { s_m[threadIdx.x / kWave] = ms.m; s_s[threadIdx.x / kWave] = ms.s; }
    __syncthreads();
    MaxSum tot;
    tot.m = s_m[0];
    tot.s = s_s[0];
    for (int w = 1; w < NT / kWave; ++w) {
        MaxSum o;
        o.m = s_m[w];
        o.s = s_s[w];
        tot = maxsum_merge(tot, o, c);
    }
    return tot;
}

template <int DTT, int DTD, int NT, int U>
__global__ __launch_bounds__(NT) void stats_kernel(SampleArgs a) {
    __shared__ float s_m[NT / kWave], s_s[NT / kWave];
    extern __shared__ RowDesc s_rows[];                       // [2 * gamma + 1]
    __shared__ int last_flag;
    __shared__ int32_t s_itmp[NT / kWave];
    __shared__ int32_t s_status;

    const int32_t g = a.gamma, NR = 2 * g + 1;
    const int32_t per_seq = (g + 1) * a.Ct + g * a.Cd;
    const int32_t b = blockIdx.x / per_seq, w = blockIdx.x % per_seq;
    MaxSum *part = a.part + (size_t)b * per_seq;
    MaxSum ms;
    if (w < (g + 1) * a.Ct) {
        const int32_t r = w / a.Ct, ch = w % a.Ct;
        const void *row = reinterpret_cast<const char *>(a.tl) +
                          ((size_t)b * (g + 1) + r) * (size_t)a.Vt * Elem<DTT>::kBytes;
        ms = chunk_maxsum<DTT, NT, U>(row, a.Vt, ch, a.Ct, a.c, s_m, s_s);
    } else {
        const int32_t w2 = w - (g + 1) * a.Ct;
        const int32_t r = w2 / a.Cd, ch = w2 % a.Cd;
        const void *row = reinterpret_cast<const char *>(a.dl) +
                          ((size_t)b * g + r) * (size_t)a.Vd * Elem<DTD>::kBytes;
        ms = chunk_maxsum<DTD, NT, U>(row, a.Vd, ch, a.Cd, a.c, s_m, s_s);
    }
    if (threadIdx.x == 0) pub(&part[w], ms);

    if (!arrive_last(&a.cnt_stats[b], (uint32_t)per_seq, &last_flag)) return;

    if (threadIdx.x == 0) s_status = 0;
    __syncthreads();
    for (int32_t r = threadIdx.x; r < NR; r += NT) {
        const bool tgt = r <= g;
        const int32_t C = tgt ? a.Ct : a.Cd;
        const MaxSum *p = tgt ? part + (size_t)r * a.Ct : part + (size_t)(g + 1) * a.Ct + (size_t)(r - g - 1) * a.Cd;
        MaxSum t = sub(&p[0]);
        for (int32_t k = 1; k < C; ++k) t = maxsum_merge(t, sub(&p[k]), a.c);
        RowDesc d;
        d.m = t.m;
        d.Z = t.s;
        d.Zk = t.s;
        d.key = 0u;
        d.tie_cut = INT32_MAX;
        d.nkept = tgt ? a.Vt : a.Vd;
        d.flags = bad_max(t.m) ? RD_NO_MASS : 0;
        d.ptok = 0.0f;
        if (d.flags & RD_NO_MASS) atomicOr(&s_status, (int)SV_SEQ_NO_MASS);
        s_rows[r] = d;
        a.rows[(size_t)b * NR + r] = d;
    }
    __syncthreads();
    const int32_t n = accept_chain<DTT, DTD, NT>(a, b, s_rows, s_itmp, &s_status);
    __syncthreads();
    if (threadIdx.x == 0) {
        SeqState st;
        st.n = n;
        st.status = s_status;
        st.pad0 = st.pad1 = 0;
        a.seq[b] = st;
        a.out_len[b] = n;
        if (a.out_status) a.out_status[b] = s_status;
    }
}

template <int DTT, int DTD, int NT>
__global__ __launch_bounds__(NT) void draw_kernel(SampleArgs a) {
    __shared__ float s_r[kTile];
    __shared__ float s_q[kTile];
    __shared__ float s_ftmp[NT / kWave];
    __shared__ double s_dtmp[NT / kWave];
    __shared__ int32_t s_itmp[NT / kWave];
    __shared__ double s_bcast[4];
    __shared__ int last_flag;

    const int32_t g = a.gamma, NR = 2 * g + 1;
    const int32_t b = blockIdx.x / a.ntiles, t = blockIdx.x % a.ntiles;
    const SeqState st = a.seq[b];
    const int32_t n = st.n;
    DrawCtx x;
    x.trow = reinterpret_cast<const char *>(a.tl) + ((size_t)b * (g + 1) + n) * (size_t)a.Vt * Elem<DTT>::kBytes;
    x.drow = n < g ? reinterpret_cast<const char *>(a.dl) + ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                   : nullptr;
    x.d2t = a.d2t;
    x.Vd = a.Vd;
    x.dp = a.rows[(size_t)b * NR + n];
    x.dq = n < g ? a.rows[(size_t)b * NR + g + 1 + n] : x.dp;
    x.c = a.c;
    x.resid = n < g;
    float *mass = a.tile_mass + (size_t)b * a.ntiles;
    const float mt = tile_mass<DTT, DTD, NT>(x, t * kTile, min(a.Vt, (t + 1) * kTile), s_r, s_q, s_ftmp);
    if (threadIdx.x == 0) pub_u32(&mass[t], __float_as_uint(mt));

    if (!arrive_last(&a.cnt_draw[b], (uint32_t)a.ntiles, &last_flag)) return;

    const double u = (double)a.u_s[b];
    int32_t tok = draw_from_tiles<DTT, DTD, NT>(x, a.Vt, mass, a.ntiles, u, s_r, s_q, s_dtmp, s_itmp, s_bcast);
    if (tok < 0 && x.resid) {
        // zero residual mass (p == q on p's support): draw from p_n itself
        x.resid = false;
        for (int32_t k = 0; k < a.ntiles; ++k) {
            const float m2 = tile_mass<DTT, DTD, NT>(x, k * kTile, min(a.Vt, (k + 1) * kTile), s_r, s_q, s_ftmp);
            if (threadIdx.x == 0) pub_u32(&mass[k], __float_as_uint(m2));
        }
        __syncthreads();
        tok = draw_from_tiles<DTT, DTD, NT>(x, a.Vt, mass, a.ntiles, u, s_r, s_q, s_dtmp, s_itmp, s_bcast);
    }
    if (threadIdx.x == 0) a.out_tokens[(size_t)b * (g + 1) + n] = tok;
}

// ---------------------------------------------------------------------------
// Host side: workspace layout and launches
// ---------------------------------------------------------------------------
int32_t stats_chunks(int32_t V, int /*dtype*/) {
    // elements per workgroup, counted as bfloat16 vectors so that the chunk
    // count depends on V only (a float32 chunk is twice the bytes)
    const int64_t per = (int64_t)kStatsThreads * kStatsUnroll * kStatsItersPerWg * 8;
    int64_t C = ((int64_t)V + per - 1) / per;
    if (C < 1) C = 1;
    if (C > kMaxChunks) C = kMaxChunks;
    return (int32_t)C;
}

bool sample_layout(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, int dt_t, int dt_d, bool topp,
                   WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *ntiles) {
    const int32_t ct = topp ? 1 : stats_chunks(Vt, dt_t);
    const int32_t cd = topp ? 1 : stats_chunks(Vd, dt_d);
    const int32_t nt = (Vt + kTile - 1) / kTile;
    const size_t NR = (size_t)(2 * gamma + 1);
    L->cnt_stats = 0;
    L->cnt_draw = align256(sizeof(uint32_t) * (size_t)B);
    L->counter_bytes = 2 * align256(sizeof(uint32_t) * (size_t)B);
    size_t off = 0;
    L->seq = off;       off = align256(off + sizeof(SeqState) * (size_t)B);
    L->rows = off;      off = align256(off + sizeof(RowDesc) * (size_t)B * NR);
    L->part = off;      off = align256(off + sizeof(MaxSum) * (size_t)B * ((size_t)(gamma + 1) * ct + (size_t)gamma * cd));
    L->kept = off;      off = align256(off + (topp ? sizeof(KeptEnt) * (size_t)B * NR * kKeptCap : 0));
    L->tile_mass = off; off = align256(off + sizeof(float) * (size_t)B * nt);
    L->data_bytes = off;
    *Ct = ct;
    *Cd = cd;
    *ntiles = nt;
    return true;
}

template <int DTT, int DTD>
static hipError_t launch_sample_dt(const SampleArgs &a, hipStream_t st) {
    const int32_t NR = 2 * a.gamma + 1;
    if (a.topp) {
        hipLaunchKernelGGL((topp_kernel<DTT, DTD, kToppThreads, kToppUnroll>), dim3(a.B * NR), dim3(kToppThreads), 0,
                           st, a);
        return hipGetLastError();
    }
    const int64_t per_seq = (int64_t)(a.gamma + 1) * a.Ct + (int64_t)a.gamma * a.Cd;
    hipLaunchKernelGGL((stats_kernel<DTT, DTD, kStatsThreads, kStatsUnroll>), dim3((unsigned)(a.B * per_seq)),
                       dim3(kStatsThreads), sizeof(RowDesc) * (size_t)NR, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((draw_kernel<DTT, DTD, kSampThreads>), dim3((unsigned)(a.B * a.ntiles)), dim3(kSampThreads), 0,
                       st, a);
    return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs &a, int dt_t, int dt_d, hipStream_t st) {
    if (dt_t == SV_BF16 && dt_d == SV_BF16) return launch_sample_dt<SV_BF16, SV_BF16>(a, st);
    if (dt_t == SV_BF16 && dt_d == SV_F32) return launch_sample_dt<SV_BF16, SV_F32>(a, st);
    if (dt_t == SV_F32 && dt_d == SV_BF16) return launch_sample_dt<SV_F32, SV_BF16>(a, st);
    return launch_sample_dt<SV_F32, SV_F32>(a, st);
}

}  // namespace sv
