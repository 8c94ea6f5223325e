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
    return exp2f((z - d.m) * c) / d.Zk;
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
__device__ void bitonic_sort_u64(uint64_t *s, int P) {
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
__device__ int32_t wg_inverse_cdf(int32_t n, G &&get, double u, bool u_is_fraction, double *s_dtmp,
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
__device__ void tile_weights(const DrawCtx &x, int32_t t0, int32_t t1, float *s_r, float *s_q) {
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
__device__ float tile_mass(const DrawCtx &x, int32_t t0, int32_t t1, float *s_r, float *s_q,
                           float *s_ftmp) {
    tile_weights<DTT, DTD, NT>(x, t0, t1, s_r, s_q);
    float acc = 0.0f;
    for (int32_t k = threadIdx.x; k < t1 - t0; k += NT) acc += s_r[k];
    return wg_sum_f32<NT>(acc, s_ftmp);
}

// Given the tile sums, find the token for u * S; returns -1 when S == 0.
template <int DTT, int DTD, int NT>
__device__ int32_t draw_from_tiles(const DrawCtx &x, int32_t V, const float *mass, int32_t ntiles,
                                   double u, float *s_r, float *s_q, double *s_dtmp,
                                   int32_t *s_itmp, double *s_bcast) {
    if (threadIdx.x == 0) {
        double S = 0.0;
        for (int32_t t = 0; t < ntiles; ++t) S += (double)mass[t];
        const double target = u * S;
        double run = 0.0, before = 0.0;
        int32_t tile = -1, lastpos = -1;
        for (int32_t t = 0; t < ntiles; ++t) {
            if (mass[t] > 0.0f) lastpos = t;
            before = run;
            run += (double)mass[t];
            if (run > target) { tile = t; break; }
        }
        if (tile < 0) { tile = lastpos; before = S - (lastpos >= 0 ? (double)mass[lastpos] : 0.0); }
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
__device__ int32_t accept_chain(const SampleArgs &a, int32_t b, const RowDesc *s_rows,
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
__device__ void topp_exact_row(const void *row, int32_t L, float m, float c, float top_p,
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
            const unsigned long long fw = (unsigned long long)((double)exp2f((z - m) * c) * kFix);
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
    const unsigned long long fws = (unsigned long long)((double)exp2f((zstar - m) * c) * kFix);
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
    d.pad = 0;
    if (d.nkept <= kKeptCap) {
        if (threadIdx.x == 0) s_nlist = 0;
        __syncthreads();
        for (int32_t j = threadIdx.x; j < L; j += NT) {
            const float z = ld_logit<DT>(row, j);
            if (row_kept(d, z, j)) {
                const int32_t pos = atomicAdd(&s_nlist, 1);
                if (pos < kKeptCap) { kept[pos].id = j; kept[pos].w = exp2f((z - m) * c); }
            }
        }
        __syncthreads();
        d.flags |= RD_HAS_LIST;
    }
    if (threadIdx.x == 0) *out = d;
}

// ---------------------------------------------------------------------------
// Top-p kernel: one workgroup per row, then the sequence epilogue.
// ---------------------------------------------------------------------------
template <int DT, int NT, int U>
__device__ void topp_row(const void *row, int32_t L, float c, float band, float top_p, RowDesc *out,
                         KeptEnt *kept, uint64_t *s_cand, unsigned char *lds_raw) {
    __shared__ uint32_t s_maxkey;
    __shared__ int32_t s_ncand;
    __shared__ float s_mred[NT / kWave], s_sred[NT / kWave];
    __shared__ double s_dtmp[NT / kWave];
    __shared__ int32_t s_itmp[NT / kWave];

    if (threadIdx.x == 0) { s_maxkey = fkey(-INFINITY); s_ncand = 0; }
    __syncthreads();

    // ---- stream: online max / sum-exp per lane, band candidates into LDS ----
    float m_l = -INFINITY, s_l = 0.0f;
    const RowSplit sp = row_split<DT>(row, L);
    using E = Elem<DT>;
    auto put = [&](float z, int32_t j) {
        const int32_t pos = atomicAdd(&s_ncand, 1);
        if (pos < kCandCap) s_cand[pos] = ((uint64_t)zkey(z) << 32) | (uint32_t)j;
    };
    auto scalar_elem = [&](float z, int32_t j) {
        // head / tail / short rows: one element at a time
        if (z > m_l) { s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2f((m_l - z) * c); m_l = z; }
        s_l += exp2f((z - m_l) * c);
        if (z > -INFINITY) {
            atomicMax(&s_maxkey, zkey(z));
            if (z >= fkey_inv(s_maxkey) - band) put(z, j);
        }
    };
    if (threadIdx.x < sp.head) scalar_elem(E::load(row, threadIdx.x), threadIdx.x);
    const u32x4 *body = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(row) +
                                                        (size_t)sp.head * E::kBytes);
    // every thread runs the same number of iterations (barrier-free, but the
    // wave-level max below needs all lanes of a wave active)
    const int32_t iters = (sp.nvec + U * NT - 1) / (U * NT);
    for (int32_t it = 0; it < iters; ++it) {
        float xv[U][E::kPerVec];
        bool have[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t v = it * U * NT + u * NT + threadIdx.x;
            have[u] = v < sp.nvec;
            u32x4 raw = have[u] ? __builtin_nontemporal_load(&body[v]) : u32x4{0, 0, 0, 0};
            E::unpack(raw, xv[u]);
        }
        float tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (have[u]) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) tm = fmaxf(tm, xv[u][k]);
            }
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2f((m_l - tm) * c);
            m_l = tm;
        }
        const float mc = m_l * c;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (have[u]) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) s_l += exp2f(fmaf(xv[u][k], c, -mc));
            }
        // share the running maximum, then collect this iteration's band members
        const float wm = wave_max(tm);
        if ((threadIdx.x & (kWave - 1)) == 0 && wm > -INFINITY) atomicMax(&s_maxkey, zkey(wm));
        const float thr = fkey_inv(s_maxkey) - band;
        if (tm >= thr) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (have[u]) {
                    const int32_t i0 = sp.head + (it * U * NT + u * NT + threadIdx.x) * E::kPerVec;
#pragma unroll
                    for (int k = 0; k < E::kPerVec; ++k)
                        if (xv[u][k] >= thr && xv[u][k] > -INFINITY) put(xv[u][k], i0 + k);
                }
        }
    }
    if (threadIdx.x < sp.tail) {
        const int32_t j = sp.head + sp.nvec * E::kPerVec + threadIdx.x;
        scalar_elem(E::load(row, j), j);
    }

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
            d.nkept = 0; d.flags = RD_NO_MASS | RD_HAS_LIST; d.pad = 0;
            *out = d;
        }
        return;
    }

    // ---- exact select inside the band ----
    const int32_t nc = s_ncand;
    const float thr_final = m - band;
    const uint32_t kthr = zkey(thr_final);
    bool fallback = nc > kCandCap;
    if (!fallback) {
        // sort key: (~key) << 32 | id ascending == logit descending, id ascending;
        // stale entries below the final threshold sort last
        const int P = pow2_at_least(nc < 2 ? 2 : nc);
        int32_t valid = 0;
        for (int32_t s = threadIdx.x; s < P; s += NT) {
            uint64_t v = ~0ull;
            if (s < nc) {
                const uint32_t k = (uint32_t)(s_cand[s] >> 32);
                const uint32_t j = (uint32_t)s_cand[s];
                if (k >= kthr) { v = ((uint64_t)(~k) << 32) | j; ++valid; }
            }
            s_cand[s] = v;
        }
        const int32_t nv = wg_sum_i32<NT>(valid, s_itmp);
        bitonic_sort_u64<NT>(s_cand, P);
        // cumulative mass in sorted order; T0 = top_p * Z
        const double T0 = (double)top_p * (double)Z;
        auto wsort = [&](int32_t s) -> float {
            const float z = fkey_inv(~(uint32_t)(s_cand[s] >> 32));
            return exp2f((z - m) * c);
        };
        const int32_t per = (nv + NT - 1) / NT;
        const int32_t s0 = min(nv, (int32_t)threadIdx.x * per), s1 = min(nv, s0 + per);
        double seg = 0.0;
        for (int32_t s = s0; s < s1; ++s) seg += (double)wsort(s);
        double M;
        const double base = wg_excl_scan_f64<NT>(seg, s_dtmp, &M);
        // the band must carry more than top_p of the mass (with a rounding margin)
        if (!(M > T0 * (1.0 + 1e-5))) fallback = true;
        if (!fallback) {
            // k = 1 + #{s <= nv - 2 : cum_incl(s) <= T0}
            int32_t cntle = 0;
            double run = base;
            for (int32_t s = s0; s < s1; ++s) {
                run += (double)wsort(s);
                if (s <= nv - 2 && run <= T0) ++cntle;
            }
            const int32_t k = 1 + wg_sum_i32<NT>(cntle, s_itmp);
            // kept mass: the cumulative at position k - 1
            double part = 0.0;
            for (int32_t s = s0; s < s1 && s < k; ++s) part += (double)wsort(s);
            double Zk;
            (void)wg_excl_scan_f64<NT>(part, s_dtmp, &Zk);
            for (int32_t s = threadIdx.x; s < k; s += NT) {
                kept[s].id = (int32_t)(uint32_t)s_cand[s];
                kept[s].w = wsort(s);
            }
            if (threadIdx.x == 0) {
                RowDesc d;
                d.m = m;
                d.Z = Z;
                d.Zk = (float)Zk;
                d.key = ~(uint32_t)(s_cand[k - 1] >> 32);
                d.tie_cut = (int32_t)(uint32_t)s_cand[k - 1];
                d.nkept = k;
                d.flags = RD_HAS_LIST;
                d.pad = 0;
                *out = d;
            }
        }
    }
    if (fallback) topp_exact_row<DT, NT>(row, L, m, c, top_p, out, kept, lds_raw);
}

// List-based draw for top-p rows: the kept ids of target row n with their
// weights, minus q_n at those ids when resid (the residual vanishes outside
// p's kept set).  Sorted by id in LDS, then the inverse CDF.
template <int DTT, int DTD, int NT>
__device__ int32_t draw_from_list(const SampleArgs &a, int32_t b, int32_t n, const RowDesc &dp,
                                  const RowDesc &dq, const KeptEnt *list, uint64_t *s_sort,
                                  double u, double *s_dtmp, int32_t *s_itmp) {
    const int32_t g = a.gamma;
    const int32_t K = dp.nkept;
    const bool resid = n < g;
    const void *drow = resid ? reinterpret_cast<const char *>(a.dl) +
                                   ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                             : nullptr;
    const int P = pow2_at_least(K < 2 ? 2 : K);
    for (int attempt = 0; attempt < 2; ++attempt) {
        const bool use_resid = resid && attempt == 0;
        __syncthreads();
        for (int32_t s = threadIdx.x; s < P; s += NT) {
            uint64_t v = ~0ull;
            if (s < K) {
                const int32_t t = list[s].id;
                float r = list[s].w / dp.Zk;
                if (use_resid) {
                    float q = 0.0f;
                    if (a.d2t) {
                        const int32_t j = lower_bound_i32(a.d2t, a.Vd, t);
                        if (j < a.Vd && a.d2t[j] == t) q = row_prob(dq, ld_logit<DTD>(drow, j), j, a.c);
                    } else {
                        q = row_prob(dq, ld_logit<DTD>(drow, t), t, a.c);
                    }
                    r = r - q > 0.0f ? r - q : 0.0f;
                }
                v = ((uint64_t)(uint32_t)t << 32) | __float_as_uint(r);
            }
            s_sort[s] = v;
        }
        bitonic_sort_u64<NT>(s_sort, P);
        double S;
        const int32_t k = wg_inverse_cdf<NT>(
            K, [&](int32_t s) { return __uint_as_float((uint32_t)s_sort[s]); }, u, true, s_dtmp, s_itmp, &S);
        if (S > 0.0) return k < 0 ? -1 : (int32_t)(s_sort[k] >> 32);
        if (!use_resid) return -1;
        // zero residual mass (only with p == q on p's support): draw from p_n
    }
    return -1;
}

template <int DTT, int DTD, int NT, int U>
__global__ __launch_bounds__(NT) void topp_kernel(SampleArgs a) {
    __shared__ uint64_t s_cand[kCandCap];
    static_assert(sizeof(RowDesc) * (2 * SV_MAX_GAMMA + 1) <= sizeof(uint64_t) * kCandCap,
                  "row descriptors must fit the candidate area");
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
    unsigned char *lds_raw = reinterpret_cast<unsigned char *>(s_cand);
    if (r <= g) {
        const void *row = reinterpret_cast<const char *>(a.tl) +
                          ((size_t)b * (g + 1) + r) * (size_t)a.Vt * Elem<DTT>::kBytes;
        topp_row<DTT, NT, U>(row, a.Vt, a.c, band, a.top_p, rows + r, kept, s_cand, lds_raw);
    } else {
        const void *row = reinterpret_cast<const char *>(a.dl) +
                          ((size_t)b * g + (r - g - 1)) * (size_t)a.Vd * Elem<DTD>::kBytes;
        topp_row<DTD, NT, U>(row, a.Vd, a.c, band, a.top_p, rows + r, kept, s_cand, lds_raw);
    }

    if (!arrive_last(&a.cnt_stats[b], (uint32_t)NR, &last_flag)) return;

    // ---- sequence epilogue: accept chain, then the draw ----
    RowDesc *s_rows = reinterpret_cast<RowDesc *>(s_cand);   // the row work is done
    for (int32_t k = threadIdx.x; k < NR; k += NT) s_rows[k] = rows[k];
    if (threadIdx.x == 0) s_status = 0;
    __syncthreads();
    for (int32_t k = threadIdx.x; k < NR; k += NT)
        if (s_rows[k].flags & RD_NO_MASS) atomicOr(&s_status, (int)SV_SEQ_NO_MASS);
    const int32_t n = accept_chain<DTT, DTD, NT>(a, b, s_rows, s_itmp, &s_status);
    const RowDesc dp = s_rows[n];
    const RowDesc dq = n < g ? s_rows[g + 1 + n] : dp;
    const double u = (double)a.u_s[b];
    __syncthreads();                                          // s_rows is reused below
    int32_t tok;
    if (dp.flags & RD_HAS_LIST) {
        tok = draw_from_list<DTT, DTD, NT>(a, b, n, dp, dq, a.kept + ((size_t)b * NR + n) * kKeptCap,
                                           s_cand, u, s_dtmp, s_itmp);
    } else {
        // kept set too large for a list: tile-by-tile over the whole row
        DrawCtx x;
        x.trow = reinterpret_cast<const char *>(a.tl) + ((size_t)b * (g + 1) + n) * (size_t)a.Vt * Elem<DTT>::kBytes;
        x.drow = n < g ? reinterpret_cast<const char *>(a.dl) + ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                       : nullptr;
        x.d2t = a.d2t;
        x.Vd = a.Vd;
        x.dp = dp;
        x.dq = dq;
        x.c = a.c;
        float *s_r = reinterpret_cast<float *>(s_cand);
        float *s_q = s_r + kTile;
        float *mass = a.tile_mass + (size_t)b * a.ntiles;
        tok = -1;
        for (int attempt = 0; attempt < 2 && tok < 0; ++attempt) {
            x.resid = n < g && attempt == 0;
            if (attempt == 1 && !(n < g)) break;
            for (int32_t t = 0; t < a.ntiles; ++t) {
                const float mt = tile_mass<DTT, DTD, NT>(x, t * kTile, min(a.Vt, (t + 1) * kTile), s_r, s_q,
                                                         reinterpret_cast<float *>(s_dtmp));
                if (threadIdx.x == 0) mass[t] = mt;
            }
            __threadfence_block();
            __syncthreads();
            tok = draw_from_tiles<DTT, DTD, NT>(x, a.Vt, mass, a.ntiles, u, s_r, s_q, s_dtmp, s_itmp, s_bcast);
        }
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
__device__ MaxSum chunk_maxsum(const void *row, int32_t L, int32_t chunk, int32_t C, float c,
                               float *s_m, float *s_s) {
    const RowSplit sp = row_split<DT>(row, L);
    const int32_t lo = (int32_t)(((int64_t)sp.nvec * chunk) / C);
    const int32_t hi = (int32_t)(((int64_t)sp.nvec * (chunk + 1)) / C);
    using E = Elem<DT>;
    float m_l = -INFINITY, s_l = 0.0f;
    auto one = [&](float z) {
        if (z > m_l) { s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2f((m_l - z) * c); m_l = z; }
        s_l += exp2f((z - m_l) * c);
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
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2f((m_l - tm) * c);
            m_l = tm;
        }
        const float mc = m_l * c;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) s_l += exp2f(fmaf(xv[u][k], c, -mc));
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
    if (threadIdx.x == 0) part[w] = ms;

    if (!arrive_last(&a.cnt_stats[b], (uint32_t)per_seq, &last_flag)) return;

    if (threadIdx.x == 0) s_status = 0;
    __syncthreads();
    for (int32_t r = threadIdx.x; r < NR; r += NT) {
        const bool tgt = r <= g;
        const int32_t C = tgt ? a.Ct : a.Cd;
        const MaxSum *p = tgt ? part + (size_t)r * a.Ct : part + (size_t)(g + 1) * a.Ct + (size_t)(r - g - 1) * a.Cd;
        MaxSum t = p[0];
        for (int32_t k = 1; k < C; ++k) t = maxsum_merge(t, p[k], a.c);
        RowDesc d;
        d.m = t.m;
        d.Z = t.s;
        d.Zk = t.s;
        d.key = 0u;
        d.tie_cut = INT32_MAX;
        d.nkept = tgt ? a.Vt : a.Vd;
        d.flags = bad_max(t.m) ? RD_NO_MASS : 0;
        d.pad = 0;
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
    if (threadIdx.x == 0) mass[t] = mt;

    if (!arrive_last(&a.cnt_draw[b], (uint32_t)a.ntiles, &last_flag)) return;

    const double u = (double)a.u_s[b];
    int32_t tok = draw_from_tiles<DTT, DTD, NT>(x, a.Vt, mass, a.ntiles, u, s_r, s_q, s_dtmp, s_itmp, s_bcast);
    if (tok < 0 && x.resid) {
        // zero residual mass (p == q on p's support): draw from p_n itself
        x.resid = false;
        for (int32_t k = 0; k < a.ntiles; ++k) {
            const float m2 = tile_mass<DTT, DTD, NT>(x, k * kTile, min(a.Vt, (k + 1) * kTile), s_r, s_q, s_ftmp);
            if (threadIdx.x == 0) mass[k] = m2;
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

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool sample_layout(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, int dt_t, int dt_d, bool topp,
                   WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *ntiles) {
    const int32_t ct = topp ? 1 : stats_chunks(Vt, dt_t);
    const int32_t cd = topp ? 1 : stats_chunks(Vd, dt_d);
    const int32_t nt = (Vt + kTile - 1) / kTile;
    const size_t NR = (size_t)(2 * gamma + 1);
    size_t off = 0;
    L->cnt_stats = off; off = align256(off + sizeof(uint32_t) * (size_t)B);
    L->cnt_draw = off;  off = align256(off + sizeof(uint32_t) * (size_t)B);
    L->seq = off;       off = align256(off + sizeof(SeqState) * (size_t)B);
    L->rows = off;      off = align256(off + sizeof(RowDesc) * (size_t)B * NR);
    L->part = off;      off = align256(off + sizeof(MaxSum) * (size_t)B * ((size_t)(gamma + 1) * ct + (size_t)gamma * cd));
    L->kept = off;      off = align256(off + (topp ? sizeof(KeptEnt) * (size_t)B * NR * kKeptCap : 0));
    L->tile_mass = off; off = align256(off + sizeof(float) * (size_t)B * nt);
    L->total = off < 256 ? 256 : off;    // never 0: 0 means invalid sizes
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
