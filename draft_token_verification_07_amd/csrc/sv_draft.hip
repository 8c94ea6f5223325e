// sv_draft.hip -- the draft-side sampler and the acceptance counters.
//
// Draft sampler ("Ling-3.0-flash-dspark" draft-model tutorial, mlqm.cn,
// sec. 4.2: the draft loop of generate() divides the logits by the
// temperature, applies _apply_top_p, takes the softmax and draws one token by
// torch.multinomial; sec. 3.1 draws draft tokens by argmax or top-p/top-k):
// one token per row of logits [B, V] from p = softmax(z / T) restricted to
// the first min(top_k, k_p) positions of the stable order (logit descending,
// lower id first), k_p being the top-p count.  The draw is the inverse CDF in
// ascending id with the caller's uniform u[b].
//
// Each row is cut into C chunks so that B * C workgroups fill the chip.  A
// chunk workgroup streams its chunk once (16-byte loads), keeps an online
// (max, sum of 2^((z - m) c)) per lane, and copies to LDS the vectors whose
// largest logit lies within a band of 8 nats (in z / T) of its running
// maximum.  It publishes (max, sum) and its band tokens as ordering codes
// (key << 32 | ~id), then arrives on the row's counter.  The last workgroup
// of the row merges the chunks in chunk order (identical results whatever
// the arrival order) and selects:
//   - neither filter on: the draw picks the chunk from the chunk masses and
//     scans that chunk's ids (a re-read of one chunk, from the caches);
//   - a cut inside the band (the usual case): the band tokens are sorted by
//     ordering code, weighed in fixed point (floor(w 2^31), exact sums), the
//     top-p count k_p is the number of prefixes with mass <= top_p Z plus one,
//     the kept set the first min(top_k, k_p) of them, and the draw is an exact
//     fixed-point inverse CDF over that list in id order;
//   - otherwise (a cut below the band, or a band too large for LDS): an exact
//     whole-row select (radix by mass for top-p, by count for top-k) and a
//     whole-row draw, by one workgroup (rare).
//
// Acceptance counters (the same page, sec. 4.2: the statistics generate()
// returns): per call, target calls, drafts proposed, drafts accepted and
// tokens emitted are added to caller-owned 64-bit counters.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

constexpr int kDraftThreads = 512;
constexpr int kDraftUnroll = 4;

// Exact count select over a whole row (one workgroup): the key K* and tie
// cut such that exactly K ids have key > K*, or key == K* and id <= tie cut
// -- the first K positions of the stable order.  8-bit digits of the key,
// most significant first, from LDS count histograms; then the tie cut, the
// need-th lowest id on K*, from contiguous id segments and a scan of their
// counts.  1 <= K <= L.
template <int DT, int NT>
__device__ SV_RARE void exact_count_select(const void *row, int32_t L, int32_t K, uint32_t *s_cnt,
                                           uint32_t *r_key, int32_t *r_tc) {
    __shared__ uint32_t s_prefix, s_need;
    __shared__ int32_t s_tc;
    __shared__ int32_t s_wsum[NT / kWave];
    if (threadIdx.x == 0) { s_prefix = 0; s_need = (uint32_t)K; s_tc = -1; }
    for (int d = 3; d >= 0; --d) {
        for (int k = threadIdx.x; k < 256; k += NT) s_cnt[k] = 0;
        __syncthreads();
        const uint32_t pre = s_prefix;
        const int hi_shift = (d + 1) * 8;
        for (int32_t j = threadIdx.x; j < L; j += NT) {
            const uint32_t key = zkey(ld_logit<DT>(row, j));
            if (d < 3 && (key >> hi_shift) != (pre >> hi_shift)) continue;
            atomicAdd(&s_cnt[(key >> (d * 8)) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t need = s_need, sel = 0;
            for (int k = 255; k >= 0; --k) {
                const uint32_t n = s_cnt[k];
                if (n >= need) { sel = (uint32_t)k; break; }
                need -= n;
            }
            s_prefix = pre | (sel << (d * 8));
            s_need = need;
        }
        __syncthreads();
    }
    const uint32_t kstar = s_prefix;
    const int32_t need = (int32_t)s_need;
    const int32_t per = (L + NT - 1) / NT;
    const int32_t j0 = min(L, (int32_t)threadIdx.x * per), j1 = min(L, j0 + per);
    int32_t cnt = 0;
    for (int32_t j = j0; j < j1; ++j) cnt += zkey(ld_logit<DT>(row, j)) == kstar ? 1 : 0;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int32_t inc = wave_incl_scan_i32(cnt);
    if (lane == kWave - 1) s_wsum[w] = inc;
    __syncthreads();
    int32_t before = inc - cnt;
    for (int k = 0; k < w; ++k) before += s_wsum[k];
    if (before < need && need <= before + cnt) {
        int32_t seen = before;
        for (int32_t j = j0; j < j1; ++j)
            if (zkey(ld_logit<DT>(row, j)) == kstar && ++seen == need) { s_tc = j; break; }
    }
    __syncthreads();
    *r_key = kstar;
    *r_tc = s_tc;
}

// Sum of the weights 2^((z - m) c) of the ids a descriptor keeps (float64).
template <int DT, int NT>
__device__ SV_RARE float kept_mass(const void *row, int32_t L, const RowDesc &d, float c, double *s_dtmp) {
    double acc = 0.0;
    for (int32_t j = threadIdx.x; j < L; j += NT) {
        const float z = ld_logit<DT>(row, j);
        if (row_kept(d, z, j)) acc += (double)exp2_hw((z - d.m) * c);
    }
    double tot;
    (void)wg_excl_scan_f64<NT>(acc, s_dtmp, &tot);
    return (float)tot;
}

// The ids of chunk ch of a row split into C chunks, as one contiguous range
// [*i0, *i1): chunk 0 also holds the head, the last chunk the tail.
__device__ __forceinline__ void chunk_ids(const RowSplit &sp, int32_t L, int32_t ch, int32_t C, int per_vec,
                                          int32_t *i0, int32_t *i1) {
    const int32_t lo = (int32_t)(((int64_t)sp.nvec * ch) / C);
    const int32_t hi = (int32_t)(((int64_t)sp.nvec * (ch + 1)) / C);
    *i0 = ch == 0 ? 0 : sp.head + lo * per_vec;
    *i1 = ch == C - 1 ? L : sp.head + hi * per_vec;
}

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void draft_kernel(DraftArgs a) {
    using E = Elem<DT>;
    constexpr int NW = NT / kWave;
    __shared__ u32x4 s_cvec[kCandVecCap];              // band vectors while streaming; later scratch
    __shared__ int32_t s_cvid[kCandVecCap];
    __shared__ uint64_t s_P[kCandCap];                 // band ordering codes
    __shared__ uint64_t s_cum[kCandCap];               // inclusive fixed-point masses in order; later scratch
    __shared__ uint32_t s_fw[kCandCap];                // fixed-point weights in order
    __shared__ uint32_t s_maxkey;
    __shared__ int32_t s_nvec, s_ncand, s_cnt2, s_tok;
    __shared__ float s_mred[NW], s_sred[NW];
    __shared__ ChunkRes s_res[kDraftMaxChunks];
    __shared__ double s_dtmp[NW];
    __shared__ int32_t s_itmp[NW];
    __shared__ int32_t s_j[2];
    __shared__ RowDesc s_desc;
    __shared__ int last_flag;
    static_assert(kTile * sizeof(float) <= sizeof(uint64_t) * kCandCap, "a draw tile fits the mass area");
    static_assert(3072 <= 16 * kCandVecCap, "radix histograms fit the vector area");

    const int32_t C = a.C;
    const int32_t b = blockIdx.x / C, ch = blockIdx.x % C;
    const int32_t L = a.V;
    const float c = a.c, band = kToppBandNats * a.T;
    const void *row = reinterpret_cast<const char *>(a.logits) + (size_t)b * (size_t)L * E::kBytes;
    const RowSplit sp = row_split<DT>(row, L);
    const int32_t lo = (int32_t)(((int64_t)sp.nvec * ch) / C);
    const int32_t hi = (int32_t)(((int64_t)sp.nvec * (ch + 1)) / C);
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;

    if (threadIdx.x == 0) { s_maxkey = fkey(-INFINITY); s_nvec = 0; s_ncand = 0; }
    __syncthreads();

    // ---- stream the chunk: online max / sum and the band vectors ----------
    float m_l = -INFINITY, s_l = 0.0f;
    auto scalar = [&](float z) {
        if (z > m_l) { s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - z) * c); m_l = z; }
        if (m_l > -INFINITY) s_l += exp2_hw((z - m_l) * c);
        if (z > -INFINITY) atomicMax(&s_maxkey, zkey(z));
    };
    if (ch == 0 && (int32_t)threadIdx.x < sp.head) scalar(E::load(row, threadIdx.x));
    if (ch == C - 1 && (int32_t)threadIdx.x < sp.tail) scalar(E::load(row, sp.head + sp.nvec * E::kPerVec + threadIdx.x));
    const u32x4 *body = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(row) +
                                                        (size_t)sp.head * E::kBytes);
    // U vectors per lane per round, all loaded before any is used; loads past
    // the chunk repeat its last vector and are masked afterwards.  The first
    // round is taken by every thread and followed by a workgroup maximum, so
    // that the band starts near the chunk maximum rather than at each lane's
    // first values (which would fill the band with early vectors).
    auto round = [&](int32_t v, bool first) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[max(lo, min(v + u * NT, hi - 1))]);
        float x[U][E::kPerVec], vm[U];
        float tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            E::unpack(raw[u], x[u]);
            const bool ok = v + u * NT < hi;
            vm[u] = -INFINITY;
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) {
                if (!ok) x[u][k] = -INFINITY;
                vm[u] = fmaxf(vm[u], x[u][k]);
            }
            tm = fmaxf(tm, vm[u]);
        }
        if (first) {
            const float wm = wave_max(tm);
            if (lane == 0 && wm > -INFINITY) atomicMax(&s_maxkey, zkey(wm));
            __syncthreads();
        }
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - tm) * c);
            m_l = tm;
        }
        if (m_l > -INFINITY) {
            const float mc = m_l * c;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) s_l += exp2_hw(fmaf(x[u][k], c, -mc));
        }
        float smax = fkey_inv(s_maxkey);
        if (tm > smax) {
            atomicMax(&s_maxkey, zkey(tm));
            smax = tm;
        }
        const float thr = smax - band;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (vm[u] >= thr && vm[u] > -INFINITY) {
                const int32_t pos = atomicAdd(&s_nvec, 1);
                if (pos < kCandVecCap) {
                    s_cvec[pos] = raw[u];
                    s_cvid[pos] = v + u * NT;
                }
            }
    };
    if (hi > lo) {
        round(lo + (int32_t)threadIdx.x, true);
        for (int32_t v = lo + (int32_t)threadIdx.x + U * NT; v < hi; v += U * NT) round(v, false);
    }
    MaxSum ms;
    ms.m = m_l;
    ms.s = s_l;
    ms = wave_maxsum_dpp(ms, c);
    if (lane == 0) { s_mred[wv] = ms.m; s_sred[wv] = ms.s; }
    __syncthreads();
    float mc_ = s_mred[0];
    for (int w = 1; w < NW; ++w) mc_ = fmaxf(mc_, s_mred[w]);
    float zc = 0.0f;
    for (int w = 0; w < NW; ++w)
        if (s_mred[w] > -INFINITY) zc += s_sred[w] * exp2_hw((s_mred[w] - mc_) * c);

    // ---- the chunk's band tokens: z >= (chunk max) - band -----------------
    const int32_t nvc = s_nvec;
    bool overflow = nvc > kCandVecCap;
    if (!overflow && mc_ > -INFINITY) {
        const float thr = mc_ - band;
        for (int32_t t0 = 0; t0 < nvc; t0 += NT) {
            const int32_t t = t0 + (int32_t)threadIdx.x;
            float x[E::kPerVec];
            int32_t i0 = 0;
            if (t < nvc) {
                E::unpack(s_cvec[t], x);
                i0 = sp.head + s_cvid[t] * E::kPerVec;
            } else {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) x[k] = -INFINITY;
            }
            uint32_t mask = 0;
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k)
                if (x[k] >= thr && x[k] > -INFINITY) mask |= 1u << k;
            int32_t pos = wave_append_n((int32_t)__popc(mask), &s_ncand);
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k)
                if ((mask >> k) & 1u) {
                    if (pos < kCandCap) s_P[pos] = pcode(zkey(x[k]), i0 + k);
                    ++pos;
                }
        }
        // head (chunk 0) and tail (last chunk) elements
        auto put = [&](bool valid, int32_t j) {
            const float z = valid ? E::load(row, j) : -INFINITY;
            const bool in = valid && z >= thr && z > -INFINITY;
            const int32_t pos = wave_append(in, &s_ncand);
            if (in && pos < kCandCap) s_P[pos] = pcode(zkey(z), j);
        };
        if (ch == 0 && sp.head > 0) put((int32_t)threadIdx.x < sp.head, threadIdx.x);
        if (ch == C - 1 && sp.tail > 0)
            put((int32_t)threadIdx.x < sp.tail, sp.head + sp.nvec * E::kPerVec + (int32_t)threadIdx.x);
    }
    __syncthreads();
    const int32_t ncand = s_ncand;
    overflow = overflow || ncand > kCandCap;

    // ---- publish the chunk, arrive on the row's counter -------------------
    if (C > 1) {
        const size_t k = (size_t)b * C + ch;
        if (!overflow)
            for (int32_t e = threadIdx.x; e < ncand; e += NT) pub_u64(&a.cand[k * kCandCap + e], s_P[e]);
        if (threadIdx.x == 0) {
            ChunkRes r;
            r.m = mc_;
            r.s = zc;
            r.n = overflow ? -1 : ncand;
            r.pad = 0;
            pub(&a.res[k], r);
        }
        if (!arrive_last(&a.counters[b], (uint32_t)C, &last_flag)) return;
        if ((int32_t)threadIdx.x < C) s_res[threadIdx.x] = sub(&a.res[(size_t)b * C + threadIdx.x]);
    } else if (threadIdx.x == 0) {
        s_res[0].m = mc_;
        s_res[0].s = zc;
        s_res[0].n = overflow ? -1 : ncand;
        s_res[0].pad = 0;
    }
    __syncthreads();

    // ---- the row: merge the chunks in chunk order -------------------------
    float m = s_res[0].m;
    bool any_over = s_res[0].n < 0;
    for (int32_t k = 1; k < C; ++k) {
        m = fmaxf(m, s_res[k].m);
        any_over = any_over || s_res[k].n < 0;
    }
    float Z = 0.0f;
    for (int32_t k = 0; k < C; ++k)
        if (s_res[k].m > -INFINITY) Z += s_res[k].s * exp2_hw((s_res[k].m - m) * c);
    const float u = a.u[b];
    int32_t tok = -1;
    float prob = 0.0f;
    int32_t status = 0;
    const bool topk_on = a.top_k > 0 && a.top_k < L;
    const bool topp_on = a.top_p < 1.0f;

    if (bad_max(m)) {
        status = SV_SEQ_NO_MASS;
    } else if (!topk_on && !topp_on) {
        // ---- no filter: the chunk from the chunk masses, then its ids -----
        if (threadIdx.x == 0) {
            double tot = 0.0;
            double sc[kDraftMaxChunks];
            for (int32_t k = 0; k < C; ++k) {
                sc[k] = s_res[k].m > -INFINITY ? (double)s_res[k].s * (double)exp2_hw((s_res[k].m - m) * c) : 0.0;
                tot += sc[k];
            }
            const double target = (double)u * tot;
            double run = 0.0;
            int32_t pick = -1, lastpos = -1;
            double before = 0.0;
            for (int32_t k = 0; k < C; ++k) {
                if (sc[k] > 0.0) { lastpos = k; before = run; }
                if (sc[k] > 0.0 && run + sc[k] > target) { pick = k; before = run; break; }
                run += sc[k];
            }
            if (pick < 0) pick = lastpos;
            s_j[0] = pick;
            s_dtmp[0] = target - before;
        }
        __syncthreads();
        const int32_t pk = s_j[0];
        const double tin = s_dtmp[0];
        __syncthreads();
        if (pk >= 0) {
            int32_t i0, i1;
            chunk_ids(sp, L, pk, C, E::kPerVec, &i0, &i1);
            double tot;
            const int32_t k = wg_inverse_cdf<NT>(
                i1 - i0, [&](int32_t s) { return exp2_hw((E::load(row, i0 + s) - m) * c); }, tin, false, s_dtmp,
                s_itmp, &tot);
            if (k >= 0) {
                tok = i0 + k;
                prob = exp2_hw((E::load(row, tok) - m) * c) / Z;
            }
        }
    } else {
        // ---- gather the row's band: every chunk's tokens with z >= m - band
        const float thr = m - band;
        bool fallback = any_over;
        int32_t nc = 0;
        if (!fallback) {
            if (threadIdx.x == 0) s_cnt2 = 0;
            __syncthreads();
            if (C > 1) {
                // one load per chunk in flight before any is used (the usual
                // band fits one round); the order of the codes is free
                int32_t nmax = 0;
                for (int32_t k = 0; k < C; ++k) nmax = max(nmax, s_res[k].n);
                const uint64_t *src = a.cand + (size_t)b * C * kCandCap;
                for (int32_t e0 = 0; e0 < nmax; e0 += NT) {
                    const int32_t e = e0 + (int32_t)threadIdx.x;
                    uint64_t Pk[kDraftMaxChunks];
#pragma unroll
                    for (int32_t k = 0; k < kDraftMaxChunks; ++k)
                        Pk[k] = (k < C && e < s_res[k].n) ? sub_u64(&src[(size_t)k * kCandCap + e]) : 0ull;
#pragma unroll
                    for (int32_t k = 0; k < kDraftMaxChunks; ++k) {
                        if (k >= C) break;                       // alike in every thread
                        const bool in = e < s_res[k].n && fkey_inv(pkey(Pk[k])) >= thr;
                        const int32_t pos = wave_append(in, &s_cnt2);
                        if (in && pos < kCandCap) s_cum[pos] = Pk[k];
                    }
                }
                __syncthreads();
                nc = s_cnt2;
                if (nc <= kCandCap)
                    for (int32_t e = threadIdx.x; e < nc; e += NT) s_P[e] = s_cum[e];
            } else {
                nc = ncand;          // one chunk: its band is the row's (same maximum)
            }
            __syncthreads();
            fallback = nc > kCandCap || nc < 1;
        }
        int32_t K = 0, P2 = 2;
        uint64_t Zkf = 0;
        bool fast_done = false;
        if (!fallback && topk_on && a.top_k <= kWave) {
            // ---- top_k <= 64: only the first 64 positions of the stable order
            // can be kept.  Each wave keeps the 64 largest ordering codes of
            // its share by in-wave bitonic networks (no workgroup barrier),
            // wave 0 merges the waves' lists and takes the weights, the top-p
            // count and the draw in registers: the arithmetic of the sorted
            // path below, on its first 64 positions.
            __shared__ uint64_t s_top[NW * kWave];
            __shared__ unsigned long long s_zk;
            __shared__ int s_fb;
            uint64_t top = 0;                                    // codes are > 0: 0 is empty
            for (int32_t e0 = wv * kWave; e0 < nc; e0 += NT) {
                const int32_t e = e0 + lane;
                top = wave_merge_top_u64(top, wave_sort_desc_u64(e < nc ? s_P[e] : 0ull));
            }
            // the waves' lists merge as a tree: wave w takes wave w + h's
            // list, h = NW / 2, NW / 4, ..., 1
            s_top[wv * kWave + lane] = top;
            __syncthreads();
#pragma unroll
            for (int h = NW / 2; h > 1; h >>= 1) {
                if (wv < h) {
                    top = wave_merge_top_u64(top, s_top[(wv + h) * kWave + lane]);
                    s_top[wv * kWave + lane] = top;
                }
                __syncthreads();
            }
            if (wv == 0) {
                const uint64_t t = wave_merge_top_u64(top, s_top[kWave + lane]);
                const int32_t nv = min(nc, (int32_t)kWave);
                const bool has = lane < nv;
                const uint32_t fw = has ? fixw32(fkey_inv(pkey(t)), m, c) : 0u;
                const uint64_t cum = wave_incl_scan_u64_dpp((uint64_t)fw);
                int32_t kp = INT32_MAX;                          // no top-p cut in the first 64
                bool fb = false;
                if (topp_on) {
                    const double T0 = (double)a.top_p * (double)Z;
                    if (!(T0 < kFixSelMaxMass)) {
                        fb = true;
                    } else {
                        const uint64_t over = __ballot(has && cum > (uint64_t)(T0 * kFixW));
                        if (over) kp = __ffsll((unsigned long long)over);
                    }
                }
                const int32_t Kf = min(a.top_k, kp);
                fb = fb || Kf > nv;
                if (!fb) {
                    const uint64_t zk = readlane_u64(cum, Kf - 1);
                    const uint64_t target = frac_floor(u, zk);
                    // entry q sums the kept weights of ids <= its own
                    const int32_t id = lane < Kf ? pid(t) : INT32_MAX;
                    uint64_t incl = 0;
                    for (int32_t j = 0; j < Kf; ++j) {
                        const int32_t idj = __builtin_amdgcn_readlane(id, j);
                        const uint32_t wj = (uint32_t)__builtin_amdgcn_readlane((int)fw, j);
                        if (idj <= id) incl += wj;
                    }
                    const uint64_t hit = __ballot(lane < Kf && fw > 0 && incl > target && incl - fw <= target);
                    const int32_t tk = hit ? __builtin_amdgcn_readlane(id, __ffsll((unsigned long long)hit) - 1) : -1;
                    if (lane == 0) {
                        s_tok = tk;
                        s_zk = zk;
                    }
                }
                if (lane == 0) s_fb = fb ? 1 : 0;
            }
            __syncthreads();
            fallback = s_fb != 0;
            fast_done = !fallback;
            if (fast_done) Zkf = s_zk;
        }
        if (!fallback && !fast_done) {
            // descending order of the ordering codes: an ascending sort with
            // zero padding, read from the top (position s is s_P[P2 - 1 - s])
            P2 = pow2_at_least(nc < 2 ? 2 : nc);
            for (int32_t e = nc + (int32_t)threadIdx.x; e < P2; e += NT) s_P[e] = 0ull;
            bitonic_sort_u64<NT>(s_P, P2);
            for (int32_t q = threadIdx.x; q < nc; q += NT) s_fw[q] = fixw32(fkey_inv(pkey(s_P[P2 - 1 - q])), m, c);
            __syncthreads();
            // inclusive masses in order (band weights are >= 2^31 e^-8 > 0, so they rise strictly)
            {
                const int32_t per = (nc + NT - 1) / NT;
                const int32_t q0 = min(nc, (int32_t)threadIdx.x * per), q1 = min(nc, q0 + per);
                uint64_t acc = 0;
                for (int32_t q = q0; q < q1; ++q) acc += s_fw[q];
                const uint64_t inc = wave_incl_scan_u64_dpp(acc);
                __shared__ uint64_t s_wtot[NW];
                if (lane == kWave - 1) s_wtot[wv] = inc;
                __syncthreads();
                uint64_t base = inc - acc;
                for (int w = 0; w < wv; ++w) base += s_wtot[w];
                for (int32_t q = q0; q < q1; ++q) { base += s_fw[q]; s_cum[q] = base; }
                if (threadIdx.x == 0) s_cnt2 = INT32_MAX;
                __syncthreads();
            }
            // top-p count k_p: positions 0..s* are kept, s* the first with a
            // mass above top_p Z; beyond the band when the band mass is not
            if (topp_on) {
                const double T0 = (double)a.top_p * (double)Z;
                if (!(T0 < kFixSelMaxMass)) {
                    fallback = true;
                } else {
                    const uint64_t T0f = (uint64_t)(T0 * kFixW);
                    for (int32_t q = threadIdx.x; q < nc; q += NT)
                        if (s_cum[q] > T0f && (q == 0 || s_cum[q - 1] <= T0f)) s_cnt2 = q + 1;
                }
                __syncthreads();
            }
            const int32_t kp = s_cnt2;                           // INT32_MAX: no top-p cut in the band
            K = topk_on ? min(a.top_k, kp) : kp;
            if (K > nc) fallback = true;
            else if (!fallback) Zkf = s_cum[K - 1];
            __syncthreads();
        }
        if (fast_done) {
            tok = s_tok;
            if (tok >= 0) prob = exp2_hw((E::load(row, tok) - m) * c) / (float)((double)Zkf / kFixW);
        } else if (!fallback) {
            // ---- the list draw: exact inverse CDF in id order over the first K
            const uint64_t target = frac_floor(u, Zkf);           // < Zkf
            if (threadIdx.x == 0) s_tok = -1;
            if (K <= NT) {
                // entry q (thread q) sums the kept weights of ids <= its own
                int32_t id = INT32_MAX;
                uint32_t w = 0;
                if ((int32_t)threadIdx.x < K) {
                    id = pid(s_P[P2 - 1 - threadIdx.x]);
                    w = s_fw[threadIdx.x];
                }
                __syncthreads();
                uint64_t incl = 0;
                if ((int32_t)threadIdx.x < K)
                    for (int32_t j = 0; j < K; ++j)
                        if (pid(s_P[P2 - 1 - j]) <= id) incl += s_fw[j];
                if ((int32_t)threadIdx.x < K && w > 0 && incl > target && incl - w <= target) s_tok = id;
                __syncthreads();
            } else {
                // sort the kept entries by id, (id << 32 | w) ascending, then a scan
                const int P3 = pow2_at_least(K);
                for (int32_t e = threadIdx.x; e < P3; e += NT)
                    s_cum[e] = e < K ? (((uint64_t)(uint32_t)pid(s_P[P2 - 1 - e]) << 32) | s_fw[e]) : ~0ull;
                bitonic_sort_u64<NT>(s_cum, P3);
                const int32_t per = (K + NT - 1) / NT;
                const int32_t q0 = min(K, (int32_t)threadIdx.x * per), q1 = min(K, q0 + per);
                uint64_t acc = 0;
                for (int32_t q = q0; q < q1; ++q) acc += (uint32_t)s_cum[q];
                const uint64_t inc = wave_incl_scan_u64_dpp(acc);
                __shared__ uint64_t s_wtot2[NW];
                if (lane == kWave - 1) s_wtot2[wv] = inc;
                __syncthreads();
                uint64_t run = inc - acc;
                for (int w = 0; w < wv; ++w) run += s_wtot2[w];
                for (int32_t q = q0; q < q1; ++q) {
                    const uint64_t w = (uint32_t)s_cum[q];
                    if (w > 0 && run <= target && target < run + w) s_tok = (int32_t)(s_cum[q] >> 32);
                    run += w;
                }
                __syncthreads();
            }
            tok = s_tok;
            if (tok >= 0) prob = exp2_hw((E::load(row, tok) - m) * c) / (float)((double)Zkf / kFixW);
        } else {
            // ---- exact whole-row select and draw (rare) ---------------------
            RowDesc d;
            d.m = m; d.Z = Z; d.Zk = Z; d.key = 0u; d.tie_cut = INT32_MAX; d.nkept = L; d.flags = 0; d.ptok = 0.0f;
            if (topp_on) {
                topp_exact_row<DT, NT, false>(row, L, m, c, a.top_p, &a.desc[b], nullptr,
                                              reinterpret_cast<unsigned char *>(s_cvec));
                __syncthreads();
                if (threadIdx.x == 0) s_desc = sub(&a.desc[b]);      // written by this thread
                __syncthreads();
                d = load_desc(&s_desc);
                __syncthreads();
            }
            if (topk_on && a.top_k < d.nkept) {
                uint32_t key;
                int32_t tc;
                exact_count_select<DT, NT>(row, L, a.top_k, reinterpret_cast<uint32_t *>(s_cvec), &key, &tc);
                d.key = key;
                d.tie_cut = tc;
                d.nkept = a.top_k;
                d.flags = 0;
                d.Zk = kept_mass<DT, NT>(row, L, d, c, s_dtmp);
            }
            DrawCtx x;
            x.trow = row;
            x.drow = nullptr;
            x.d2t = nullptr;
            x.Vd = L;
            x.dp = d;
            x.dq = d;
            x.c = c;
            x.resid = false;
            tok = draw_row_one_wg<DT, DT, NT>(x, L, kTile, (double)u, reinterpret_cast<float *>(s_cum), s_dtmp,
                                              s_itmp, s_j);
            if (tok >= 0) prob = row_prob(d, E::load(row, tok), tok, c);
        }
    }
    if (threadIdx.x == 0) {
        a.out_tokens[b] = (tok >= 0 && a.d2t) ? a.d2t[tok] : tok;
        if (a.out_prob) a.out_prob[b] = prob;
        if (a.out_status) a.out_status[b] = status;
    }
}

// ---------------------------------------------------------------------------
// Acceptance counters: one pass over accept_len, integer sums added to the
// caller's counters with 64-bit atomics (exact, any order).
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(NT) void count_kernel(const int32_t *len, int32_t B, int32_t gamma,
                                                   unsigned long long *ctr) {
    constexpr int NW = NT / kWave;
    __shared__ uint64_t s_v[3][NW];
    uint64_t nvalid = 0, acc = 0, bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < B; i += (int64_t)gridDim.x * NT) {
        const int32_t n = len[i];
        if (n < 0 || n > gamma) {
            ++bad;
        } else {
            ++nvalid;
            acc += (uint64_t)n;
        }
    }
    nvalid = wave_total_u64(nvalid);
    acc = wave_total_u64(acc);
    bad = wave_total_u64(bad);
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    if (lane == 0) { s_v[0][wv] = nvalid; s_v[1][wv] = acc; s_v[2][wv] = bad; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t0 = 0, t1 = 0, t2 = 0;
        for (int w = 0; w < NW; ++w) { t0 += s_v[0][w]; t1 += s_v[1][w]; t2 += s_v[2][w]; }
        if (t0) {
            atomicAdd(&ctr[0], (unsigned long long)t0);
            atomicAdd(&ctr[1], (unsigned long long)(t0 * (uint64_t)gamma));
            atomicAdd(&ctr[3], (unsigned long long)(t1 + t0));
        }
        if (t1) atomicAdd(&ctr[2], (unsigned long long)t1);
        if (t2) atomicAdd(&ctr[4], (unsigned long long)t2);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

hipError_t launch_draft(const DraftArgs &a, int dtype, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.B * a.C));
    if (dtype == SV_BF16)
        hipLaunchKernelGGL((draft_kernel<SV_BF16, kDraftThreads, kDraftUnroll>), grid, dim3(kDraftThreads), 0, st, a);
    else
        hipLaunchKernelGGL((draft_kernel<SV_F32, kDraftThreads, kDraftUnroll>), grid, dim3(kDraftThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_count(const int32_t *accept_len, int32_t B, int32_t gamma, unsigned long long *counters,
                        hipStream_t st) {
    constexpr int NT = 256;
    int64_t g = ((int64_t)B + NT * 4 - 1) / (NT * 4);
    if (g < 1) g = 1;
    if (g > 256) g = 256;
    hipLaunchKernelGGL((count_kernel<NT>), dim3((unsigned)g), dim3(NT), 0, st, accept_len, B, gamma, counters);
    return hipGetLastError();
}

}  // namespace sv
