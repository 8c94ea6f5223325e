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
//   top-p on:  one kernel (topp_kernel).  One workgroup per row (target and
//     draft rows) streams the row once, keeping the online max / sum-exp per
//     lane and copying to LDS the 16-byte vectors whose largest logit lies
//     within a band of the running maximum.  It then selects the kept set in
//     exact fixed-point arithmetic: the band's tokens are binned by their
//     distance below the row maximum, the bin whose inclusive mass first
//     exceeds top_p * Z is found by a scan, and only that bin's tokens are
//     ranked by (logit desc, id asc) -- the page's _apply_top_p order -- to
//     find the last kept token.  The row publishes its kept set (boundary
//     key, tie cut, kept mass, kept ids and weights).  The last workgroup of
//     each sequence to arrive on the sequence's counter runs the accept chain
//     and draws from the kept lists (a few dozen ids), so the rows are read
//     once.  Rows the bins cannot settle take sub-band or radix selects, and
//     rows whose band does not hold top_p of the mass take an exact radix
//     select over the whole row.
//   top-p off: three kernels in a row on the stream; each kernel boundary is
//     the only synchronisation.  (1) stats_kernel: rows are cut into chunks,
//     each workgroup streams one chunk and writes its (max, sum-exp), and one
//     probe workgroup per sequence reads the logits at the draft tokens.
//     (2) tile_kernel: one workgroup per (sequence, tile of target ids)
//     merges the chunk results in chunk order, runs the accept chain, and
//     sums the fixed-point residual (or bonus) weights of its tile of target
//     row n.  (3) pick_kernel: one workgroup per sequence finds the tile
//     holding u_s * S and the token inside it.
#include <math.h>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

// Three 512-thread top-p workgroups per CU (24 waves, so at most 80 VGPRs)
// keep every row of a 64 x 11-row batch resident at once.
#define SV_TOPP_OCCUPANCY __attribute__((amdgpu_waves_per_eu(6)))

// ---------------------------------------------------------------------------
// Top-p kernel: one workgroup per row, then the sequence epilogue.
// ---------------------------------------------------------------------------

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
// Top-p select over the band by bins (the usual case).  The band tokens are
// binned by their distance below the row maximum: kWave bins of equal width,
// so a lower bin holds only larger logits and equal logits share a bin.  Per-bin
// fixed-point mass and count give, by a scan that every wave runs alike, the
// bin holding the boundary; only that bin's tokens are ranked against each
// other.  The kept set is every band token whose ordering code is at least
// the boundary's -- the set the general path finds.  Five workgroup barriers.
// Returns false, having written nothing to global memory and left the band
// vectors in LDS, when the row needs the general path.
constexpr int kBinMembers = 224;        // tokens of the boundary bin ranked here

struct BinSelectLds {
    uint64_t *P;          // [kCandCap] ordering codes of the band tokens
    uint32_t *fw;         // [kCandCap] their fixed-point weights
    uint64_t *bm;         // [kWave] bin masses (zero on entry)
    uint32_t *bc;         // [kWave] bin counts (zero on entry)
    uint64_t *mP;         // [kBinMembers] the boundary bin's tokens
    uint32_t *mfw;        // [kBinMembers]
    int32_t *cnt;         // [3] tokens, boundary-bin tokens, kept entries (zero on entry)
    uint64_t *res;        // [3] boundary code (zero on entry), kept mass, kept count
    float *ptok;          // zero on entry
};

template <int DT, int NT>
__device__ __forceinline__ bool bin_select(const void *row, const RowSplit &sp, int32_t L, int32_t nvc,
                                           const u32x4 *s_cvec, const int32_t *s_cvid, const BinSelectLds &l,
                                           float m, float Z, float c, float band, float top_p, int32_t xtok,
                                           const int32_t *d2t, RowDesc *out, KeptEnt *kept) {
    using E = Elem<DT>;
    constexpr int NB = kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const double T0 = (double)top_p * (double)Z;
    if (!(T0 < kFixSelMaxMass)) return false;
    const uint64_t T0f = (uint64_t)(T0 * kFixW);
    const float thr = m - band;
    const float bscale = (float)NB / band;
    auto bin_of = [&](float z) { return (int)fminf((m - z) * bscale, (float)(NB - 1)); };
    // A. band tokens as (logit bits, id): one band vector per thread, its
    // tokens in consecutive slots; -0 is folded onto +0 so that the ordering
    // code below orders values
    auto put = [&](int32_t pos, float z, int32_t id) {
        if (pos < kCandCap) l.P[pos] = ((uint64_t)__float_as_uint(z + 0.0f) << 32) | (uint32_t)id;
    };
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
        int32_t pos = wave_append_n((int32_t)__popc(mask), &l.cnt[0]);
#pragma unroll
        for (int k = 0; k < E::kPerVec; ++k)
            if ((mask >> k) & 1u) put(pos++, x[k], i0 + k);
    }
    if (sp.head + sp.tail > 0) {
        // elements outside the vector body (rows not 16-byte aligned)
        const int32_t i = threadIdx.x;
        const bool v = i < sp.head + sp.tail;
        const int32_t j = i < sp.head ? i : sp.head + sp.nvec * E::kPerVec + (i - sp.head);
        const float z = v ? E::load(row, j) : -INFINITY;
        const bool in = v && z >= thr && z > -INFINITY;
        const int32_t pos = wave_append(in, &l.cnt[0]);
        if (in) put(pos, z, j);
    }
    __syncthreads();
    // ordering codes, fixed-point weights and bin totals, one token per thread
    const int32_t n = l.cnt[0];
    if (n > kCandCap) return false;
    for (int32_t t = threadIdx.x; t < n; t += NT) {
        const uint64_t r = l.P[t];
        const float z = __uint_as_float((uint32_t)(r >> 32));
        const uint32_t fw = fixw32(z, m, c);
        l.P[t] = pcode(fkey(z), (int32_t)(uint32_t)r);
        l.fw[t] = fw;
        const int bn = bin_of(z);
        atomicAdd(reinterpret_cast<unsigned long long *>(&l.bm[bn]), (unsigned long long)fw);
        atomicAdd(&l.bc[bn], 1u);
    }
    __syncthreads();

    // B. the boundary bin, in every wave alike: the first bin whose inclusive
    // mass exceeds T0 (the band must hold more than T0, with the margin of the
    // general path); then its tokens, compacted
    const uint64_t bm = l.bm[lane];
    const int32_t bc = (int32_t)l.bc[lane];
    const uint64_t binc = wave_incl_scan_u64_dpp(bm);
    const int32_t cinc = wave_incl_scan_i32(bc);
    const uint64_t total = readlane_u64(binc, kWave - 1);
    if (!((double)total > (double)T0f * (1.0 + 1e-5))) return false;
    const int bstar = __ffsll((unsigned long long)__ballot(binc > T0f)) - 1;
    const uint64_t before = readlane_u64(binc - bm, bstar);
    const int32_t cbefore = __builtin_amdgcn_readlane(cinc - bc, bstar);
    const int32_t nmem = __builtin_amdgcn_readlane(bc, bstar);
    if (nmem > kBinMembers) return false;
    for (int32_t t0 = 0; t0 < n; t0 += NT) {
        const int32_t t = t0 + (int32_t)threadIdx.x;
        uint64_t P = 0;
        bool in = false;
        if (t < n) {
            P = l.P[t];
            in = bin_of(fkey_inv(pkey(P))) == bstar;
        }
        const int32_t pos = wave_append(in, &l.cnt[1]);
        if (in && pos < kBinMembers) {
            l.mP[pos] = P;
            l.mfw[pos] = l.fw[t];
        }
    }
    __syncthreads();

    // C. the boundary token: the mass strictly ahead of it <= T0 < that plus
    // its own weight (exactly one token of the bin)
    const int32_t nm = l.cnt[1];
    if (nm != nmem) return false;                 // by construction equal
    if ((int32_t)threadIdx.x < nm) {
        const uint64_t Pi = l.mP[threadIdx.x];
        const uint64_t wi = l.mfw[threadIdx.x];
        uint64_t ahead = before;
        int32_t cnt = 0;
        for (int32_t j = 0; j < nm; ++j)
            if (l.mP[j] > Pi) {
                ahead += l.mfw[j];
                ++cnt;
            }
        if (ahead <= T0f && ahead + wi > T0f) {
            l.res[0] = Pi;
            l.res[1] = ahead + wi;
            l.res[2] = (uint64_t)(cbefore + cnt + 1);
        }
    }
    __syncthreads();

    // D. publish: the kept list (order free), the draft token's probability,
    // then the row descriptor
    const uint64_t pmin = l.res[0];
    if (pmin == 0) return false;                  // by construction found
    const float Zk = (float)((double)l.res[1] / kFixW);
    for (int32_t t0 = 0; t0 < n; t0 += NT) {
        const int32_t t = t0 + (int32_t)threadIdx.x;
        const uint64_t P = t < n ? l.P[t] : 0ull;
        const bool in = t < n && P >= pmin;
        const int32_t pos = wave_append(in, &l.cnt[2]);
        if (in) {
            const int32_t id = pid(P);
            KeptEnt e;
            e.id = id;
            e.w = exp2_hw((fkey_inv(pkey(P)) - m) * c);
            pub(&kept[pos], e);
            if (xtok >= 0 && (d2t ? d2t[id] == xtok : id == xtok)) *l.ptok = e.w / Zk;
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
        d.nkept = (int32_t)l.res[2];
        d.flags = RD_HAS_LIST;
        d.ptok = *l.ptok;
        pub(out, d);
    }
    return true;
}

template <int DT, int NT, int U>
__device__ __forceinline__ void topp_row(const void *row, int32_t L, float c, float band, float top_p, RowDesc *out,
                                         KeptEnt *kept, uint64_t *s_lds, int32_t *s_cvid, int32_t xtok,
                                         const int32_t *d2t) {
    __shared__ uint32_t s_maxkey;
    __shared__ int32_t s_ncand, s_nvec, s_nsel, s_nk, s_nlist;
    __shared__ float s_mred[NT / kWave], s_sred[NT / kWave];
    __shared__ unsigned long long s_bmass[4], s_zk, s_pmin;
    __shared__ float s_ptok;
    __shared__ int32_t s_bcnt[3];
    __shared__ unsigned long long s_bres[3];
    uint64_t *s_cand = s_lds;                                          // [kCandCap] band tokens
    u32x4 *s_cvec = reinterpret_cast<u32x4 *>(s_lds + kCandCap);       // [kCandVecCap] band vectors
    uint64_t *s_P = s_lds + kCandCap;                                  // [kCandCap] after expansion
    uint32_t *s_fw = reinterpret_cast<uint32_t *>(s_lds + 2 * kCandCap);            // [kCandCap]
    uint64_t *s_ahead = s_lds + 2 * kCandCap + kCandCap / 2;                        // [NT] / radix bins

    if (threadIdx.x == 0) { s_maxkey = fkey(-INFINITY); s_ncand = 0; s_nvec = 0; s_nlist = 0; s_ptok = 0.0f; }
    if (threadIdx.x < 3) { s_bcnt[threadIdx.x] = 0; s_bres[threadIdx.x] = 0; }
    if (threadIdx.x < kWave) {                  // bin select: masses and counts
        s_ahead[threadIdx.x] = 0;
        reinterpret_cast<uint32_t *>(s_ahead + kWave)[threadIdx.x] = 0;
    }
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
    // Elements are taken from the raw vectors where they are used (one
    // shift or mask each), so only the U raw vectors are held per lane.
    auto tile = [&](const u32x4 (&raw)[U], const float (&vm)[U], float tm, int32_t vbase, int nu) {
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - tm) * c);
            m_l = tm;
        }
        const float mc = m_l * c;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < nu) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) s_l += exp2_hw(fmaf(E::elem(raw[u], k), c, -mc));
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
    auto vec_max = [&](const u32x4 &r) {
        float v = E::elem(r, 0);
#pragma unroll
        for (int k = 1; k < E::kPerVec; ++k) v = fmaxf(v, E::elem(r, k));
        return v;
    };
    // A partial iteration (the first or the last): the loads are issued
    // unconditionally at clamped indices (a load under a divergent branch is
    // waited for inside it, one round trip per vector); vectors past the row
    // (the last U - nu) are left out afterwards.  Requires sp.nvec >= 1.
    auto load_iter = [&](int32_t it, u32x4 (&raw)[U], float (&vm)[U], float &tm) -> int {
        const int32_t vbase = it * U * NT + threadIdx.x;
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[min(vbase + u * NT, sp.nvec - 1)]);
        int nu = 0;
        tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = vbase + u * NT < sp.nvec;
            vm[u] = ok ? vec_max(raw[u]) : -INFINITY;
            tm = fmaxf(tm, vm[u]);
            nu += ok ? 1 : 0;
        }
        return nu;
    };
    const int32_t full = sp.nvec / (U * NT);
    const int32_t iters = (sp.nvec + U * NT - 1) / (U * NT);
    if (iters > 0) {
        // iteration 0: take the workgroup-wide maximum first, so the band
        // starts near the row maximum instead of each lane's own tile maximum
        u32x4 raw[U];
        float vm[U], tm;
        const int nu = load_iter(0, raw, vm, tm);
        const float wm = wave_max(tm);
        if ((threadIdx.x & (kWave - 1)) == 0 && wm > -INFINITY) atomicMax(&s_maxkey, zkey(wm));
        __syncthreads();
        tile(raw, vm, tm, threadIdx.x, nu);
    }
    // Waves with more of their row left issue first, so that rows sharing a
    // CU finish together instead of oldest-first: level floor(4 (full - it) /
    // (full + 1)), i.e. the number of k in 1..3 with it <= lim_k (no division
    // in the loop).
    int prio = -1;
    const int32_t lim1 = full - (1 * (full + 1) + 3) / 4;
    const int32_t lim2 = full - (2 * (full + 1) + 3) / 4;
    const int32_t lim3 = full - (3 * (full + 1) + 3) / 4;
    for (int32_t it = 1; it < full; ++it) {
        {
            const int lvl = (it <= lim1) + (it <= lim2) + (it <= lim3);
            if (lvl != prio) {
                prio = lvl;
                if (lvl >= 3) __builtin_amdgcn_s_setprio(3);
                else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
                else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
        }
        const int32_t vbase = it * U * NT + threadIdx.x;
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[vbase + u * NT]);
        float vm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) vm[u] = vec_max(raw[u]);
        float tm = vm[0];
#pragma unroll
        for (int u = 1; u < U; ++u) tm = fmaxf(tm, vm[u]);
        tile(raw, vm, tm, vbase, U);
    }
    if (iters > full && full > 0) {
        u32x4 raw[U];
        float vm[U], tm;
        const int nu = load_iter(full, raw, vm, tm);
        tile(raw, vm, tm, full * U * NT + threadIdx.x, nu);
    }
    if (threadIdx.x < sp.tail) scalar_elem(E::load(row, sp.head + sp.nvec * E::kPerVec + threadIdx.x));
    // What follows is short and on the critical path, while other workgroups
    // on this CU are still streaming: issue ahead of their waves.
    __builtin_amdgcn_s_setprio(3);

    // ---- row max and mass ----
    MaxSum ms;
    ms.m = m_l;
    ms.s = s_l;
    ms = wave_maxsum_dpp(ms, c);
    if ((threadIdx.x & (kWave - 1)) == 0) { s_mred[threadIdx.x / kWave] = ms.m; s_sred[threadIdx.x / kWave] = ms.s; }
    __syncthreads();
    float m = s_mred[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) m = fmaxf(m, s_mred[w]);
    float Z = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const float mw = s_mred[w];
        if (mw > -INFINITY) Z += s_sred[w] * exp2_hw((mw - m) * c);
    }
    if (bad_max(m)) {
        if (threadIdx.x == 0) {
            RowDesc d;
            d.m = m; d.Z = 0.0f; d.Zk = 0.0f; d.key = 0xffffffffu; d.tie_cut = -1;
            d.nkept = 0; d.flags = RD_NO_MASS | RD_HAS_LIST; d.ptok = 0.0f;
            pub(out, d);
        }
        return;
    }

    const float thr_final = m - band;
    const int32_t nvc = s_nvec;
    // ---- usual case: select by bins ----
    if (nvc <= kCandVecCap) {
        BinSelectLds l;
        l.P = s_cand;
        l.fw = s_fw;
        l.bm = s_ahead;
        l.bc = reinterpret_cast<uint32_t *>(s_ahead + kWave);
        l.mP = s_ahead + kWave + kWave / 2;
        l.mfw = reinterpret_cast<uint32_t *>(l.mP + kBinMembers);
        l.cnt = s_bcnt;
        l.res = reinterpret_cast<uint64_t *>(s_bres);
        l.ptok = &s_ptok;
        static_assert(kWave + kWave / 2 + kBinMembers + kBinMembers / 2 <= 512, "bins fit the pairwise area");
        static_assert(kCandCap + 2 * kCandVecCap <= 2 * kCandCap, "band vectors stay clear of the token lists");
        if (bin_select<DT, NT>(row, sp, L, nvc, s_cvec, s_cvid, l, m, Z, c, band, top_p, xtok, d2t, out, kept))
            return;
        __syncthreads();      // the general path below reuses what the bin select wrote
    }

    // ---- expand the band: every token with z >= m - band ----
    bool fallback = nvc > kCandVecCap;
    if (!fallback) {
        // called by every lane of every wave (wave-aggregated append)
        auto put = [&](bool valid, float z, int32_t j) {
            const bool in = valid && z >= thr_final && z > -INFINITY;
            const int32_t pos = wave_append(in, &s_ncand);
            if (in && pos < kCandCap) s_cand[pos] = ((uint64_t)zkey(z) << 32) | (uint32_t)j;
        };
        // one vector per thread: its in-band elements take consecutive slots
        // (one LDS atomic per wave)
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
            uint32_t mask = 0;
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k)
                if (x[k] >= thr_final && x[k] > -INFINITY) mask |= 1u << k;
            int32_t pos = wave_append_n((int32_t)__popc(mask), &s_ncand);
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k)
                if ((mask >> k) & 1u) {
                    if (pos < kCandCap) s_cand[pos] = ((uint64_t)zkey(x[k]) << 32) | (uint32_t)(i0 + k);
                    ++pos;
                }
        }
        if (sp.head > 0) {
            const bool vh = threadIdx.x < (unsigned)sp.head;
            put(vh, vh ? E::load(row, threadIdx.x) : -INFINITY, threadIdx.x);
        }
        if (sp.tail > 0) {
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
#pragma unroll 8
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
                                                  const KeptEnt *pre_list, const KeptEnt *pre_qlist,
                                                  uint64_t *s_lds, double u, double *s_dtmp, int32_t *s_itmp) {
    // pre_list / pre_qlist: copies of the lists already in LDS, or null
    const int32_t g = a.gamma;
    const int32_t K = dp.nkept;
    const bool resid = n < g;
    const void *drow = resid ? reinterpret_cast<const char *>(a.dl) +
                                   ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes
                             : nullptr;
    // q's kept list in LDS as an open-addressing hash table from target id
    // to q (at most half full), so each p entry finds its q in a probe or two
    const int32_t Kq = (resid && (dq.flags & RD_HAS_LIST) && dq.nkept <= kQListCap) ? dq.nkept : -1;
    constexpr int kHash = 2 * kQListCap;
    int32_t *s_hid = reinterpret_cast<int32_t *>(s_lds);                     // [kHash], -1 = empty
    float *s_hq = reinterpret_cast<float *>(s_lds) + kHash;                  // [kHash]
    uint64_t *s_work = s_lds + kHash;                                        // past the table
    auto hslot = [](int32_t id) { return (int32_t)(((uint32_t)id * 0x9E3779B1u) >> 21) & (kHash - 1); };
    // one round trip for both lists: this thread's p entry and q entries
    KeptEnt e;
    e.id = INT32_MAX;
    e.w = 0.0f;
    if (K <= NT && (int32_t)threadIdx.x < K) e = pre_list ? pre_list[threadIdx.x] : sub(&list[threadIdx.x]);
    constexpr int kQPer = (kQListCap + NT - 1) / NT;
    KeptEnt qe[kQPer];
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
        const int32_t j = (int32_t)threadIdx.x + k * NT;
        if (j < Kq) qe[k] = pre_qlist ? pre_qlist[j] : sub(&qlist[j]);
    }
    if (Kq >= 0) {
        for (int32_t i = threadIdx.x; i < kHash; i += NT) s_hid[i] = -1;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kQPer; ++k) {
            const int32_t j = (int32_t)threadIdx.x + k * NT;
            if (j < Kq) {
                const int32_t id = a.d2t ? a.d2t[qe[k].id] : qe[k].id;
                int32_t sl = hslot(id);
                while (atomicCAS(&s_hid[sl], -1, id) != -1) sl = (sl + 1) & (kHash - 1);
                s_hq[sl] = qe[k].w / dq.Zk;
            }
        }
    }
    __syncthreads();
    auto weight = [&](const KeptEnt &pe, bool use_resid) -> float {
        float r = pe.w / dp.Zk;
        if (use_resid) {
            float q = 0.0f;
            if (Kq >= 0) {
                // ids within a list are distinct; the table is never full
                for (int32_t sl = hslot(pe.id);; sl = (sl + 1) & (kHash - 1)) {
                    const int32_t h = s_hid[sl];
                    if (h == pe.id) {
                        q = s_hq[sl];
                        break;
                    }
                    if (h == -1) break;
                }
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
#pragma unroll 8
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
// is too large for a list); one workgroup (rarely taken).
template <int DTT, int DTD, int NT>
__device__ SV_RARE int32_t draw_full_row(const SampleArgs &a, int32_t b, int32_t n, const RowDesc &dp,
                                         const RowDesc &dq, double u, float *s_w, double *s_dtmp, int32_t *s_itmp,
                                         int32_t *s_j) {
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
    x.resid = n < g;
    int32_t tok = draw_row_one_wg<DTT, DTD, NT>(x, a.Vt, a.tile, u, s_w, s_dtmp, s_itmp, s_j);
    if (tok < 0 && x.resid) {
        // zero residual mass: draw from p_n itself
        x.resid = false;
        tok = draw_row_one_wg<DTT, DTD, NT>(x, a.Vt, a.tile, u, s_w, s_dtmp, s_itmp, s_j);
    }
    return tok;
}

// The draw of draw_from_list when both kept lists are in LDS with at most
// kWave entries each, for 512-thread workgroups: p's entry i is handled by
// the 8 threads of one half-row (threads 8i .. 8i+7), thread s of them taking
// every 8th entry from s of the other list; their parts combine by DPP inside
// the half-row.  Two workgroup barriers (three with a d2t map).  The
// arithmetic is that of draw_from_list, so both give the same token.
__device__ __forceinline__ float half_row_sum_f32(float v) {
    v = dpp_add_f32<0xB1, 0xf>(v);     // quad_perm [1,0,3,2]
    v = dpp_add_f32<0x4E, 0xf>(v);     // quad_perm [2,3,0,1]
    v = dpp_add_f32<0x141, 0xf>(v);    // row_half_mirror
    return v;
}
__device__ __forceinline__ uint64_t half_row_sum_u64(uint64_t v) {
    v = dpp_add_u64<0xB1, 0xf>(v);
    v = dpp_add_u64<0x4E, 0xf>(v);
    v = dpp_add_u64<0x141, 0xf>(v);
    return v;
}

template <int NT>
__device__ __forceinline__ int32_t group_draw_list(const SampleArgs &a, const RowDesc &dp, const RowDesc &dq,
                                                   bool resid, const KeptEnt *pl, const KeptEnt *pq, double u,
                                                   uint64_t *s_rf, int32_t *s_id, int32_t *s_qid, int32_t *s_tok) {
    constexpr int G = 8;
    static_assert(NT == G * kWave, "one half-row per entry of a 64-entry list");
    const int32_t i = threadIdx.x / G, sl = threadIdx.x % G;
    const int32_t K = dp.nkept, Kq = resid ? dq.nkept : 0;
    const bool has = i < K;
    KeptEnt e;
    e.id = INT32_MAX;
    e.w = 0.0f;
    if (has) e = pl[i];
    if (threadIdx.x == 0) *s_tok = -1;
    if (a.d2t && Kq > 0) {
        // q's entries carry draft ids: their target ids once, in LDS
        if ((int32_t)threadIdx.x < Kq) s_qid[threadIdx.x] = a.d2t[pq[threadIdx.x].id];
        __syncthreads();
    }
    // q of entry i: at most one of q's entries has its id (ids are distinct)
    float qpart = 0.0f;
#pragma unroll
    for (int it = 0; it < kWave / G; ++it) {
        const int32_t j = sl + it * G;
        if (has && j < Kq) {
            const KeptEnt qe = pq[j];
            const int32_t qid = a.d2t ? s_qid[j] : qe.id;
            if (qid == e.id) qpart = qe.w / dq.Zk;
        }
    }
    const float q = half_row_sum_f32(qpart);
    for (int attempt = 0; attempt < 2; ++attempt) {
        const bool use_resid = resid && attempt == 0;
        float r = e.w / dp.Zk;
        if (use_resid) r = r - q > 0.0f ? r - q : 0.0f;
        const uint64_t rf = has ? (uint64_t)((double)r * kFixW) : 0ull;
        if (sl == 0) {
            s_rf[i] = rf;
            s_id[i] = e.id;
        }
        __syncthreads();
        // mass of the entries with id <= this entry's, and the total
        uint64_t inc = 0, S = 0;
#pragma unroll
        for (int it = 0; it < kWave / G; ++it) {
            const int32_t j = sl + it * G;
            if (j < K) {
                const uint64_t rj = s_rf[j];
                S += rj;
                if (s_id[j] <= e.id) inc += rj;
            }
        }
        inc = half_row_sum_u64(inc);
        S = half_row_sum_u64(S);
        if (S > 0) {
            // exactly one entry (in id order) brackets the target
            const uint64_t target = (uint64_t)(u * (double)S);
            if (has && sl == 0 && rf > 0 && inc > target && inc - rf <= target) *s_tok = e.id;
            __syncthreads();
            return *s_tok;
        }
        if (!use_resid) return -1;
        // zero residual mass (only with p == q on p's support): draw from p_n
        __syncthreads();
    }
    return -1;
}

// Kept-list prefixes staged by the sequence epilogue, at the end of the
// band area (past what the draws use).
constexpr int kPreBase = 4096;                 // u64 offset in the band area
constexpr int kPreSlots = 1536;                // list entries (8 bytes each)
constexpr int kPreMax = 64;                    // entries per row at most

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
    static_assert(2 * kQListCap + kKeptCap <= kPreBase, "q table and list sort stay below the list prefixes");
    static_assert(2 * kQListCap + NT / 2 + NT + 1 <= kPreBase, "q table and pairwise draw stay below the prefixes");
    static_assert(kPreBase + kPreSlots <= 2 * kCandCap + kCandCap / 2 + 512, "list prefixes fit the band area");
    static_assert(kPreSlots / (2 * SV_MAX_GAMMA + 1) >= 1, "every row gets a prefix slot");
    static_assert(kTile * sizeof(float) <= sizeof(uint64_t) * 4096, "draw tiles must fit the band area");
    __shared__ int last_flag;
    __shared__ int32_t s_itmp[NT / kWave];
    __shared__ double s_dtmp[NT / kWave];
    __shared__ int32_t s_j[2];

    const int32_t g = a.gamma, NR = 2 * g + 1;
    const int32_t b = blockIdx.x / NR, r = blockIdx.x % NR;
    const float band = kToppBandNats * a.T;
    RowDesc *rows = a.rows + (size_t)b * NR;
    KeptEnt *kept = a.kept + ((size_t)b * NR + r) * a.kept_stride;
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
        // Draft row i checks slice i of the map (SSD guide sec. 6: strictly
        // increasing target ids in [0, Vt)); the gamma slices cover every
        // entry and step, and the epilogue reports a violation as SV_SEQ_D2T.
        int map_bad = 0;
        if (map) {
            const int32_t i = r - g - 1;
            const int32_t j0 = (int32_t)((int64_t)a.Vd * i / g), j1 = (int32_t)((int64_t)a.Vd * (i + 1) / g);
            int bad = 0;
            for (int32_t j = j0 + (int32_t)threadIdx.x; j < j1; j += NT) {
                const int32_t cur = map[j], prev = j > 0 ? map[j - 1] : -1;
                bad |= (cur < 0 || cur >= a.Vt || cur <= prev) ? 1 : 0;
            }
            map_bad = __syncthreads_or(bad);
        }
        if constexpr (DTT == DTD) {
            topp_row<DTT, NT, U>(row, tgt ? a.Vt : a.Vd, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
        } else {
            if (tgt)
                topp_row<DTT, NT, U>(row, a.Vt, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
            else
                topp_row<DTD, NT, U>(row, a.Vd, a.c, band, a.top_p, rows + r, kept, s_cand, s_cvid, xt, map);
        }
        if (map_bad && threadIdx.x == 0) {
            // thread 0 published the descriptor: mark it
            RowDesc d = sub(rows + r);
            d.flags |= RD_BAD_MAP;
            pub(rows + r, d);
        }
    }

    if (!arrive_last(&a.cnt_stats[b], (uint32_t)NR, &last_flag)) return;

    // ---- sequence epilogue: accept chain, then the draw ----
    // one round of loads: the row descriptors, the kept-list prefixes, each
    // wave's copy of the first kWave draft positions (token, uniform) and the
    // sampling uniform
    RowDesc *s_rows = reinterpret_cast<RowDesc *>(s_cand);   // the row work is done
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int32_t *x = a.tokens + (size_t)b * g;
    const int32_t ti = lane < g ? x[lane] : 0;
    const double ui = lane < g ? (double)a.u_acc[(size_t)b * g + lane] : 0.0;
    const double u = (double)a.u_s[b];
    for (int32_t k = threadIdx.x; k < NR; k += NT) s_rows[k] = sub(&rows[k]);
    // the first kPre entries of every row's kept list, loaded in the same
    // round (entries past a row's own count are stale and never used)
    KeptEnt *s_pre = reinterpret_cast<KeptEnt *>(s_cand + kPreBase);
    const int32_t kPre = min(kPreMax, kPreSlots / NR);
    for (int32_t e = threadIdx.x; e < NR * kPre; e += NT)
        s_pre[e] = sub(&a.kept[((size_t)b * NR + e / kPre) * a.kept_stride + min(e % kPre, a.kept_stride - 1)]);
    __syncthreads();
    // Status and chain, in every wave alike (so that all waves take the same
    // branch below): every row has published the probability of its own
    // draft token; n is the first position where u * q < p fails.
    int32_t status = 0, n = g;
    {
        uint64_t nomass = 0, badmap = 0;
        for (int32_t k0 = 0; k0 < NR; k0 += kWave) {
            const int32_t k = k0 + lane;
            nomass |= __ballot(k < NR && (s_rows[k].flags & RD_NO_MASS) != 0);
            badmap |= __ballot(k < NR && (s_rows[k].flags & RD_BAD_MAP) != 0);
        }
        if (nomass) status |= SV_SEQ_NO_MASS;
        if (badmap) status |= SV_SEQ_D2T;
        for (int32_t i0 = 0; i0 < g; i0 += kWave) {
            const int32_t i = i0 + lane;
            int32_t t = ti;
            double uu = ui;
            if (i0 > 0) {                                   // more than kWave drafts (rare)
                t = i < g ? x[i] : 0;
                uu = i < g ? (double)a.u_acc[(size_t)b * g + i] : 0.0;
            }
            bool bad = false, rej = false;
            if (i < g) {
                bad = t < 0 || t >= a.Vt;
                const float pa = s_rows[i].ptok, qc = s_rows[g + 1 + i].ptok;
                if (wv == 0) {
                    if (a.out_p) a.out_p[(size_t)b * g + i] = pa;
                    if (a.out_q) a.out_q[(size_t)b * g + i] = qc;
                }
                rej = !(uu * (double)qc < (double)pa);
            }
            if (__ballot(bad)) status |= SV_SEQ_TOKEN_RANGE;
            const uint64_t rb = __ballot(rej);
            if (rb && n == g) n = i0 + __ffsll((unsigned long long)rb) - 1;
        }
        if (wv == 0)
            for (int32_t i0 = 0; i0 <= g; i0 += kWave) {
                const int32_t i = i0 + lane;
                if (i <= g && i != n) a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? (i0 == 0 ? ti : x[i]) : -1;
            }
    }
    const RowDesc dp = s_rows[n];
    const RowDesc dq = n < g ? s_rows[g + 1 + n] : dp;
    int32_t tok = -1;
    const bool short_lists = (dp.flags & RD_HAS_LIST) && dp.nkept <= kPre && dp.nkept <= kWave &&
                             (n == g || ((dq.flags & RD_HAS_LIST) && dq.nkept <= kPre && dq.nkept <= kWave));
    __syncthreads();                                          // s_rows is reused below
    bool drawn = false;
    if constexpr (NT == 8 * kWave) {
        if (short_lists) {
            // usual case: both lists are in LDS with at most kWave entries
            uint64_t *s_rf = s_cand;                                         // [kWave]
            int32_t *s_id = reinterpret_cast<int32_t *>(s_cand + kWave);     // [kWave]
            int32_t *s_qid = s_id + kWave;                                   // [kWave]
            static_assert(kWave + kWave <= kPreBase, "draw scratch stays below the list prefixes");
            tok = group_draw_list<NT>(a, dp, dq, n < g, s_pre + (size_t)n * kPre,
                                      s_pre + (size_t)(n < g ? g + 1 + n : n) * kPre, u, s_rf, s_id, s_qid, &s_j[0]);
            drawn = true;
        }
    }
    if (!drawn) {
        if (dp.flags & RD_HAS_LIST) {
            const KeptEnt *pl = dp.nkept <= kPre ? s_pre + (size_t)n * kPre : nullptr;
            const KeptEnt *pq = (n < g && dq.nkept <= kPre) ? s_pre + (size_t)(g + 1 + n) * kPre : nullptr;
            tok = draw_from_list<DTT, DTD, NT>(a, b, n, dp, dq, a.kept + ((size_t)b * NR + n) * a.kept_stride,
                                               a.kept + ((size_t)b * NR + g + 1 + n) * a.kept_stride, pl, pq, s_cand,
                                               u, s_dtmp, s_itmp);
        } else {
            // kept set too large for a list: tile-by-tile over the whole row
            tok = draw_full_row<DTT, DTD, NT>(a, b, n, dp, dq, u, reinterpret_cast<float *>(s_cand), s_dtmp, s_itmp,
                                              s_j);
        }
    }
    if (threadIdx.x == 0) {
        a.out_tokens[(size_t)b * (g + 1) + n] = tok;
        a.out_len[b] = n;
        if (a.out_status) a.out_status[b] = status;
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
    // U vectors per lane per round, all loaded before any is used.  The loads
    // are unconditional (past the chunk they repeat its last vector, and the
    // values are masked to -inf afterwards): a load under a branch would be
    // waited for inside the branch, one round trip per vector.
    for (int32_t v = lo + threadIdx.x; v < hi; v += U * NT) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[min(v + u * NT, hi - 1)]);
        float xv[U][E::kPerVec];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            E::unpack(raw[u], xv[u]);
            if (v + u * NT >= hi) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) xv[u][k] = -INFINITY;
            }
        }
        float tm = xv[0][0];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) tm = fmaxf(tm, xv[u][k]);
        if (tm > m_l) {
            s_l = (m_l == -INFINITY) ? 0.0f : s_l * exp2_hw((m_l - tm) * c);
            m_l = tm;
        }
        if (m_l > -INFINITY) {
            const float mc = m_l * c;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) s_l += exp2_hw(fmaf(xv[u][k], c, -mc));
        }
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

// The logits at each draft token of sequence b (target row i at x_i, draft
// row i at x_i's draft id), read while the chunk workgroups stream, so the
// chain needs no loads of its own.  With d2t, groups of G lanes search the map
// for the tokens' draft ids, 64 / G tokens per wave at once.
template <int DTT, int DTD, int NT, int G>
__device__ __forceinline__ void probe_tokens_g(const SampleArgs &a, int32_t b) {
    constexpr int TPW = kWave / G, TPB = (NT / kWave) * TPW;
    const int32_t g = a.gamma;
    const int gl = threadIdx.x & (G - 1);
    for (int32_t base = 0; base < g; base += TPB) {
        const int32_t i = base + (int32_t)(threadIdx.x / G);
        const bool has = i < g;
        const int32_t t = has ? a.tokens[(size_t)b * g + i] : -1;
        const bool valid = has && t >= 0 && t < a.Vt;
        const void *trow = reinterpret_cast<const char *>(a.tl) +
                           ((size_t)b * (g + 1) + (has ? i : 0)) * (size_t)a.Vt * Elem<DTT>::kBytes;
        const void *drow = reinterpret_cast<const char *>(a.dl) +
                           ((size_t)b * g + (has ? i : 0)) * (size_t)a.Vd * Elem<DTD>::kBytes;
        Probe pr;
        pr.zt = 0.0f;
        pr.zd = -INFINITY;
        if (valid && gl == 0) pr.zt = ld_logit<DTT>(trow, t);
        if (a.d2t) {
            const int32_t j = group_lower_bound<G>(a.d2t, a.Vd, valid ? t : 0);
            if (valid && gl == 0 && j < a.Vd && a.d2t[j] == t) pr.zd = ld_logit<DTD>(drow, j);
        } else if (valid && gl == 0) {
            pr.zd = ld_logit<DTD>(drow, t);
        }
        if (has && gl == 0) a.probe[(size_t)b * g + i] = pr;
    }
}

template <int DTT, int DTD, int NT>
__device__ __forceinline__ void probe_tokens(const SampleArgs &a, int32_t b) {
    // the widest groups that still cover every token in one pass
    constexpr int W = NT / kWave;
    const int32_t g = a.gamma;
    if (!a.d2t || g > 2 * W * 8) probe_tokens_g<DTT, DTD, NT, 8>(a, b);
    else if (g <= W) probe_tokens_g<DTT, DTD, NT, 64>(a, b);
    else if (g <= 2 * W) probe_tokens_g<DTT, DTD, NT, 32>(a, b);
    else if (g <= 4 * W) probe_tokens_g<DTT, DTD, NT, 16>(a, b);
    else probe_tokens_g<DTT, DTD, NT, 8>(a, b);
}

// Draft-id boundaries of the draw tiles under d2t: jb[k] = the first j with
// d2t[j] >= k * tile, k = 0..ntiles.  Entry j (0 <= j <= Vd) owns the k with
// d2t[j-1] < k * tile <= d2t[j] (d2t[-1] = -1, d2t[Vd] = +inf); the probe
// workgroup of sequence b takes the j in [b (Vd+1) / B, (b+1) (Vd+1) / B).
//
// The same pass checks the map (SSD guide sec. 6: d2t sends draft id j to a
// distinct target id; this library takes it strictly increasing in
// [0, Vt)): entry j must lie in [0, Vt) and above entry j - 1.  The B slices
// cover every entry and every step once; a violation sets the call's map
// flag, which the draw tiles turn into SV_SEQ_D2T on every sequence.
template <int NT>
__device__ __forceinline__ void tile_bounds(const SampleArgs &a, int32_t b) {
    const int64_t n1 = (int64_t)a.Vd + 1;
    const int32_t j0 = (int32_t)(n1 * b / a.B), j1 = (int32_t)(n1 * (b + 1) / a.B);
    bool bad = false;
    for (int32_t j = j0 + (int32_t)threadIdx.x; j < j1; j += NT) {
        const int64_t prev = j > 0 ? (int64_t)a.d2t[j - 1] : -1;
        const int64_t cur = j < a.Vd ? (int64_t)a.d2t[j] : INT64_MAX;
        if (j < a.Vd && (cur < 0 || cur >= a.Vt || cur <= prev)) bad = true;
        const int64_t klo = prev < 0 ? 0 : prev / a.tile + 1;
        int64_t khi = cur / a.tile;
        if (khi > a.ntiles) khi = a.ntiles;
        for (int64_t k = klo; k <= khi; ++k) a.tile_jb[k] = j;
    }
    if (bad && a.gamma > 0) atomicOr(a.map_flag, 1u);
}

// Plain mode, first launch.  Grid: B probe workgroups, then
// B * ((gamma+1) * Ct + gamma * Cd) chunk workgroups; each chunk workgroup
// writes the (max, sum) of its chunk, each probe workgroup the logits at the
// draft tokens (and, with d2t, its share of the tile boundaries).  The next
// launch merges them.
template <int DTT, int DTD, int NT, int U>
__global__ __launch_bounds__(NT) void stats_kernel(SampleArgs a) {
    __shared__ float s_m[NT / kWave], s_s[NT / kWave];
    const int32_t g = a.gamma;
    const int32_t per_seq = (g + 1) * a.Ct + g * a.Cd;
    if ((int32_t)blockIdx.x < a.B) {
        const int32_t b = blockIdx.x;
        probe_tokens<DTT, DTD, NT>(a, b);
        if (a.d2t) tile_bounds<NT>(a, b);
        return;
    }
    const int32_t b = ((int32_t)blockIdx.x - a.B) / per_seq;
    const int32_t w = ((int32_t)blockIdx.x - a.B) % per_seq;
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
    if (threadIdx.x == 0) a.part[(size_t)b * per_seq + w] = ms;
}

// ---------------------------------------------------------------------------
// Plain-mode draw.  Grid: B * ntiles; tile k covers target ids
// [k * tile, (k+1) * tile), read with the row's 16-byte vectors (a vector that
// straddles two tiles is read by both, each keeping its own ids).  Weights are
// taken in fixed point, F(w) = floor(w * 2^52): tile masses and every prefix
// are exact integers, so the pass that picks a tile and the pass that searches
// inside it agree exactly whatever the order of the additions, and the draw
// target floor(u * S) is exact.  Residual weights are F(max(0, p_t - q_t));
// q_t comes from the draft row's vectors when it is laid out like the target
// row, from a d2t scatter through LDS, or from single loads.  pick_kernel
// (one workgroup per sequence) then picks the tile and searches it.
// ---------------------------------------------------------------------------

// floor(w * 2^52) for 0 <= w < 2^11, from the bits of w (exact, no float64).
__device__ __forceinline__ uint64_t fix52(float w) {
    const uint32_t bits = __float_as_uint(w);
    const int e = (int)((bits >> 23) & 0xffu);
    const uint64_t m = (uint64_t)((bits & 0x7fffffu) | (e ? 0x800000u : 0u));
    const int sh = (e ? e : 1) - 98;                 // w = m * 2^(e - 150), times 2^52
    if (sh >= 0) return m << sh;
    return sh > -24 ? m >> -sh : 0;
}

// One tile of a plain-mode draw, loaded: the vectors of target ids [t0, t1)
// (U per thread, slice u = vectors v_lo + u * NT + tid), the draft values
// where they come with the same vectors, and q of mapped ids in LDS.
template <int DTT, int DTD, int NT>
struct DrawTile {
    using ET = Elem<DTT>;
    using ED = Elem<DTD>;
    static constexpr int U = kTile / ET::kPerVec / NT + 1;
    const void *trow, *drow;
    RowSplit sp;
    int32_t t0, t1, v_lo, v_hi;
    float mp, izp, mq, izq, c;
    bool resid, fused, mapped, nomass;
    u32x4 rt[U], rd[U];

    // Weight of target id t (fixed point) given its target logit and q.
    // Contraction is off in both: the tile pass and the pick must compute the
    // same float for every id, whether q arrives through LDS or inline.
    __device__ __forceinline__ uint64_t weight_q(float zt, float q) const {
#pragma clang fp contract(off)
        const float p = nomass ? 0.0f : exp2_hw((zt - mp) * c) * izp;
        if (!resid) return fix52(p);
        return fix52(p - q > 0.0f ? p - q : 0.0f);
    }
    __device__ __forceinline__ float qprob(float zq) const {
#pragma clang fp contract(off)
        return exp2_hw((zq - mq) * c) * izq;
    }

    // q of target id t when it does not come with the vectors
    __device__ __forceinline__ float q_single(int32_t t, const float *s_q) const {
        if (!resid) return 0.0f;
        if (mapped) return s_q[t - t0];
        return qprob(ED::load(drow, t));
    }
    // weights of the ids in slice u's vector of this thread, summed; f(t, w) per id
    template <typename F>
    __device__ __forceinline__ uint64_t slice(int u, const float *s_q, F &&f) const {
        const int32_t v = v_lo + u * NT + (int32_t)threadIdx.x;
        uint64_t s = 0;
        if (v < v_hi) {
            float zt[ET::kPerVec], zq[ET::kPerVec];
            ET::unpack(rt[u], zt);
            if constexpr (DTT == DTD) {
                if (fused) ET::unpack(rd[u], zq);
            }
            const int32_t i0 = sp.head + v * ET::kPerVec;
#pragma unroll
            for (int k = 0; k < ET::kPerVec; ++k) {
                const int32_t t = i0 + k;
                if (t < t0 || t >= t1) continue;
                float q = 0.0f;
                if (resid) {
                    if constexpr (DTT == DTD) q = fused ? qprob(zq[k]) : q_single(t, s_q);
                    else q = q_single(t, s_q);
                }
                const uint64_t w = weight_q(zt[k], q);
                f(t, w);
                s += w;
            }
        }
        return s;
    }
    // Slice u's vector when all its ids lie in [t0, t1) and in one subtile
    // (2^sh ids): *sidx gets the subtile and *sum the weights' sum, and the
    // per-id range checks and subtile bookkeeping of slice() are skipped.
    // Returns false, with nothing done, for any other vector.
    __device__ __forceinline__ bool slice_block(int u, const float *s_q, int sh, int *sidx, uint64_t *sum) const {
        const int32_t v = v_lo + u * NT + (int32_t)threadIdx.x;
        const int32_t i0 = sp.head + v * ET::kPerVec;
        if (!(v < v_hi && i0 >= t0 && i0 + ET::kPerVec <= t1 &&
              ((i0 - t0) >> sh) == ((i0 + ET::kPerVec - 1 - t0) >> sh)))
            return false;
        float zt[ET::kPerVec], zq[ET::kPerVec];
        ET::unpack(rt[u], zt);
        if constexpr (DTT == DTD) {
            if (fused) ET::unpack(rd[u], zq);
        }
        uint64_t s = 0;
#pragma unroll
        for (int k = 0; k < ET::kPerVec; ++k) {
            float q = 0.0f;
            if (resid) {
                if constexpr (DTT == DTD) q = fused ? qprob(zq[k]) : q_single(i0 + k, s_q);
                else q = q_single(i0 + k, s_q);
            }
            s += weight_q(zt[k], q);
        }
        *sidx = (i0 - t0) >> sh;
        *sum = s;
        return true;
    }
    // the ids of [t0, t1) outside the vector body (head or tail), one per
    // thread: thread i takes the i-th of them
    __device__ __forceinline__ int32_t edge_id() const {
        const int32_t i = (int32_t)threadIdx.x;
        const int32_t hb = max(t0, 0), he = min(t1, sp.head);          // head ids in the tile
        const int32_t nh = he > hb ? he - hb : 0;
        if (i < nh) return hb + i;
        const int32_t tb = max(t0, sp.head + sp.nvec * ET::kPerVec), te = t1;
        const int32_t ntl = te > tb ? te - tb : 0;
        if (i - nh < ntl) return tb + (i - nh);
        return -1;
    }
};

// Row pointers, modes and normalisers of a draw over target row n.
template <int DTT, int DTD, int NT>
__device__ __forceinline__ void draw_tile_params(DrawTile<DTT, DTD, NT> &x, const SampleArgs &a, int32_t b,
                                                 int32_t n, const RowDesc &dp, const RowDesc &dq) {
    using ET = Elem<DTT>;
    using ED = Elem<DTD>;
    const int32_t g = a.gamma;
    x.trow = reinterpret_cast<const char *>(a.tl) + ((size_t)b * (g + 1) + n) * (size_t)a.Vt * ET::kBytes;
    x.drow = n < g ? reinterpret_cast<const char *>(a.dl) + ((size_t)b * g + n) * (size_t)a.Vd * ED::kBytes
                   : nullptr;
    x.resid = n < g;
    x.mapped = x.resid && a.d2t != nullptr;
    x.sp = row_split<DTT>(x.trow, a.Vt);
    x.fused = false;
    if constexpr (DTT == DTD)
        if (x.resid && !x.mapped) x.fused = row_split<DTD>(x.drow, a.Vd).head == x.sp.head;
    x.c = a.c;
    x.mp = dp.m;
    x.izp = 1.0f / dp.Zk;
    x.nomass = (dp.flags & RD_NO_MASS) != 0;
    x.mq = dq.m;
    x.izq = (dq.flags & RD_NO_MASS) ? 0.0f : 1.0f / dq.Zk;
}

template <int DTT, int DTD, int NT>
__device__ __forceinline__ void draw_tile_load(DrawTile<DTT, DTD, NT> &x, const SampleArgs &a, int32_t b,
                                               int32_t n, const RowDesc &dp, const RowDesc &dq, int32_t k,
                                               int32_t j0, int32_t j1, float *s_q) {
    using ET = Elem<DTT>;
    using ED = Elem<DTD>;
    draw_tile_params<DTT, DTD, NT>(x, a, b, n, dp, dq);
    x.t0 = k * a.tile;
    x.t1 = min(a.Vt, x.t0 + a.tile);
    const int32_t body0 = x.sp.head, body1 = x.sp.head + x.sp.nvec * ET::kPerVec;
    x.v_lo = x.t0 <= body0 ? 0 : (x.t0 - body0) / ET::kPerVec;
    x.v_hi = x.t1 <= body0 ? 0 : min(x.sp.nvec, (min(x.t1, body1) - body0 + ET::kPerVec - 1) / ET::kPerVec);
    const u32x4 *tb = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x.trow) +
                                                      (size_t)x.sp.head * ET::kBytes);
    // every load of the tile before any use (one round trip); indices are
    // clamped into the tile's vectors and out-of-tile ids dropped when used
    if (x.v_hi > x.v_lo) {
#pragma unroll
        for (int u = 0; u < DrawTile<DTT, DTD, NT>::U; ++u)
            x.rt[u] = __builtin_nontemporal_load(&tb[min(x.v_lo + u * NT + (int32_t)threadIdx.x, x.v_hi - 1)]);
        // keep these loads ahead of the draft-side loads below: the d2t
        // scatter waits for those, and by then these must have arrived too
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DTT == DTD) {
            if (x.fused) {
                const u32x4 *db = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x.drow) +
                                                                  (size_t)x.sp.head * ED::kBytes);
#pragma unroll
                for (int u = 0; u < DrawTile<DTT, DTD, NT>::U; ++u)
                    x.rd[u] = __builtin_nontemporal_load(&db[min(x.v_lo + u * NT + (int32_t)threadIdx.x, x.v_hi - 1)]);
            }
        }
    }
    if (x.mapped) {
        // q of the mapped draft ids [j0, j1) (at most tile of them) into s_q
        constexpr int UJ = kTile / NT;
        int32_t tj[UJ];
        float zq[UJ];
        const bool any = j1 > j0;
        if (any) {
#pragma unroll
            for (int u = 0; u < UJ; ++u) {
                const int32_t j = min(j0 + u * NT + (int32_t)threadIdx.x, j1 - 1);
                tj[u] = a.d2t[j];
                zq[u] = ED::load(x.drow, j);
            }
        }
        for (int32_t i = threadIdx.x; i < x.t1 - x.t0; i += NT) s_q[i] = 0.0f;
        __syncthreads();
        if (any) {
#pragma unroll
            for (int u = 0; u < UJ; ++u) {
                const int32_t j = j0 + u * NT + (int32_t)threadIdx.x;
                const int32_t i = tj[u] - x.t0;
                if (j < j1 && i >= 0 && i < x.t1 - x.t0) s_q[i] = x.qprob(zq[u]);
            }
        }
        __syncthreads();
    }
}

// Plain mode, second launch.  Grid: B * ntiles.  Workgroup (b, k) merges the
// chunk statistics of sequence b in chunk order (every workgroup of b alike),
// runs the accept chain, and sums the fixed-point residual (or bonus)
// weights of target tile k of row n.  Workgroup (b, 0) also writes the
// accepted tokens, the probabilities, the status and the sequence state.
template <int DTT, int DTD, int NT>
__global__ __launch_bounds__(NT) void tile_kernel(SampleArgs a) {
    using DT = DrawTile<DTT, DTD, NT>;
    constexpr int U = DT::U;
    constexpr int NW = NT / kWave;
    static_assert(NT > SV_MAX_GAMMA, "one thread per draft position");
    extern __shared__ RowDesc s_rows[];                       // [2 * gamma + 1]
    constexpr int kTilePartCap = 256;                         // partials staged in LDS (else read twice)
    __shared__ MaxSum s_part[kTilePartCap];
    __shared__ float s_q[kTile];
    __shared__ uint64_t s_sub[kSubTiles];

    const int32_t g = a.gamma, NR = 2 * g + 1;
    const int32_t per_seq = (g + 1) * a.Ct + g * a.Cd;
    const int32_t b = blockIdx.x / a.ntiles, k = blockIdx.x % a.ntiles;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    if ((int)threadIdx.x < kSubTiles) s_sub[threadIdx.x] = 0;

    // one round of loads: the chunk partials (into LDS), this thread's draft
    // position (token, probe, uniform), the tile's draft-id range
    const MaxSum *part = a.part + (size_t)b * per_seq;
    const bool staged = per_seq <= kTilePartCap;
    if (staged)
        for (int32_t q = threadIdx.x; q < per_seq; q += NT) s_part[q] = part[q];
    const int32_t i = threadIdx.x;
    int32_t t = -1;
    Probe pr;
    pr.zt = 0.0f;
    pr.zd = -INFINITY;
    double ua = 0.0;
    if (i < g) {
        t = a.tokens[(size_t)b * g + i];
        pr = a.probe[(size_t)b * g + i];
        ua = (double)a.u_acc[(size_t)b * g + i];
    }
    int32_t j0 = 0, j1 = 0;
    uint32_t map_bad = 0;
    if (a.d2t) {
        j0 = min(max(a.tile_jb[k], 0), a.Vd);
        j1 = min(max(a.tile_jb[k + 1], j0), a.Vd);
        if (k == 0 && threadIdx.x == 0) map_bad = a.map_flag[0];
    }
    __syncthreads();
    // Rows of few chunks are merged by one thread each, chunk by chunk in
    // order; rows of many by one wave each (lane l folds chunks l, l + 64, ...
    // in order, then the lanes combine by DPP).  Either way the pattern is fixed
    // by the row's chunk count, so identical rows give identical results.
    auto put_row = [&](int32_t r, const MaxSum &acc) {
        RowDesc d;
        d.m = acc.m;
        d.Z = acc.s;
        d.Zk = acc.s;
        d.key = 0u;
        d.tie_cut = INT32_MAX;
        d.nkept = r <= g ? a.Vt : a.Vd;
        d.flags = bad_max(acc.m) ? RD_NO_MASS : 0;
        d.ptok = 0.0f;
        s_rows[r] = d;
    };
    constexpr int32_t kSerialChunks = 8;
    auto row_chunks = [&](int32_t r, int32_t &C, int32_t &off) {
        const bool tgt = r <= g;
        C = tgt ? a.Ct : a.Cd;
        off = tgt ? r * a.Ct : (g + 1) * a.Ct + (r - g - 1) * a.Cd;
    };
    for (int32_t r = threadIdx.x; r < NR; r += NT) {
        int32_t C, off;
        row_chunks(r, C, off);
        if (C > kSerialChunks) continue;
        MaxSum acc = staged ? s_part[off] : part[off];
        for (int32_t q = 1; q < C; ++q) acc = maxsum_merge(acc, staged ? s_part[off + q] : part[off + q], a.c);
        put_row(r, acc);
    }
    if (a.Ct > kSerialChunks || a.Cd > kSerialChunks) {
        for (int32_t r = wv; r < NR; r += NW) {
            int32_t C, off;
            row_chunks(r, C, off);
            if (C <= kSerialChunks) continue;                // wave-uniform
            MaxSum acc;
            acc.m = -INFINITY;
            acc.s = 0.0f;
            for (int32_t q = lane; q < C; q += kWave)
                acc = maxsum_merge(acc, staged ? s_part[off + q] : part[off + q], a.c);
            acc = wave_maxsum_dpp(acc, a.c);
            if (lane == 0) put_row(r, acc);
        }
    }
    __syncthreads();
    // the chain: n is the first position where u * q < p fails (exactly:
    // both products fit a double)
    float pa = 0.0f, qc = 0.0f;
    bool bad = false, rej = false;
    if (i < g) {
        if (t < 0 || t >= a.Vt) {
            bad = true;
        } else {
            pa = row_prob(s_rows[i], pr.zt, t, a.c);
            qc = row_prob(s_rows[g + 1 + i], pr.zd, t, a.c);
        }
        rej = !(ua * (double)qc < (double)pa);
    }
    int32_t n;
    {
        // positions 0..g-1 live in the first waves; every wave reads them from LDS
        __shared__ unsigned long long s_rej[(SV_MAX_GAMMA + kWave) / kWave];
        __shared__ int s_flags;
        if (threadIdx.x == 0) s_flags = 0;
        const uint64_t rb = __ballot(rej);
        if (lane == 0 && wv * kWave < g) s_rej[wv] = rb;
        __syncthreads();
        if (bad) atomicOr(&s_flags, 1);
        n = g;
        for (int w = 0; w * kWave < g; ++w)
            if (s_rej[w]) {
                n = w * kWave + __ffsll(s_rej[w]) - 1;
                break;
            }
        if (k == 0) {
            if (i < g) {
                if (a.out_p) a.out_p[(size_t)b * g + i] = pa;
                if (a.out_q) a.out_q[(size_t)b * g + i] = qc;
            }
            if (i <= g && i != n) a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? t : -1;
        }
        __syncthreads();
        if (k == 0 && threadIdx.x == 0) {
            int32_t status = (s_flags & 1) ? SV_SEQ_TOKEN_RANGE : 0;
            if (map_bad) status |= SV_SEQ_D2T;
            for (int32_t r = 0; r < NR; ++r)
                if (s_rows[r].flags & RD_NO_MASS) status |= SV_SEQ_NO_MASS;
            SeqState st;
            st.n = n;
            st.status = status;
            st.pad0 = st.pad1 = 0;
            st.dp = s_rows[n];
            st.dq = s_rows[n < g ? g + 1 + n : n];
            a.seq[b] = st;
            a.out_len[b] = n;
            if (a.out_status) a.out_status[b] = status;
        }
    }
    const RowDesc dp = s_rows[n];
    const RowDesc dq = n < g ? s_rows[g + 1 + n] : dp;
    DT x;
    draw_tile_load<DTT, DTD, NT>(x, a, b, n, dp, dq, k, j0, j1, s_q);
    // masses by subtile (kSubTiles equal id ranges of the tile, in id order);
    // a vector's ids fall in at most two subtiles
    const int sh = __builtin_ctz((unsigned)(a.tile / kSubTiles));
    int cur = -1;
    uint64_t acc = 0;
    auto flush = [&]() {
        if (cur >= 0 && acc) atomicAdd(reinterpret_cast<unsigned long long *>(&s_sub[cur]), (unsigned long long)acc);
    };
    auto add = [&](int32_t tt, uint64_t w) {
        const int sidx = (tt - x.t0) >> sh;
        if (sidx != cur) {
            flush();
            cur = sidx;
            acc = 0;
        }
        acc += w;
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int sidx;
        uint64_t sum;
        if (x.slice_block(u, s_q, sh, &sidx, &sum)) {
            if (sidx != cur) {
                flush();
                cur = sidx;
                acc = 0;
            }
            acc += sum;
        } else {
            (void)x.slice(u, s_q, add);
        }
    }
    flush();
    const int32_t te = x.edge_id();
    if (te >= 0) {
        const uint64_t w = x.weight_q(Elem<DTT>::load(x.trow, te), x.q_single(te, s_q));
        if (w) atomicAdd(reinterpret_cast<unsigned long long *>(&s_sub[(te - x.t0) >> sh]), (unsigned long long)w);
    }
    __syncthreads();
    if (wv == 0) {
        static_assert(kSubTiles == kWave, "one subtile per lane of the first wave");
        const uint64_t v = s_sub[lane];
        a.tile_sub[((size_t)b * a.ntiles + k) * kSubTiles + lane] = v;
        const uint64_t mass = wave_total_u64(v);
        if (lane == 0) a.tile_mass[(size_t)b * a.ntiles + k] = mass;
    }
}

// Plain mode, third launch.  Grid: B.  Workgroup b picks the tile holding
// floor(u * S) from the tile masses, reloads it and finds the token inside
// (exact fixed-point sums, so the pick and the search agree).
template <int DTT, int DTD, int NT>
__global__ __launch_bounds__(NT) void pick_kernel(SampleArgs a) {
    using DT = DrawTile<DTT, DTD, NT>;
    constexpr int NW = NT / kWave;
    __shared__ float s_q[kTile];                  // rare fallback (zero residual mass)
    __shared__ uint64_t s_tmp[NW];
    __shared__ int32_t s_qj[kWave];               // draft id of each target id of the subtile (d2t)
    __shared__ uint64_t s_pick[2];                // picked tile, offset of floor(u * S) inside it
    __shared__ uint64_t s_sp[2];                  // picked subtile, offset inside it
    __shared__ int32_t s_jr[2];
    __shared__ int32_t s_tok;
    // rare fallback (zero residual mass)
    __shared__ double s_dtmp[NW];
    __shared__ int32_t s_itmp[NW];
    __shared__ int32_t s_j[2];

    const int32_t g = a.gamma;
    const int32_t b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    // every draw tile has read the map flag (previous launch): clear it for the next call
    if (b == 0 && threadIdx.x == 0 && a.d2t) a.map_flag[0] = 0u;
    const SeqState *st = &a.seq[b];
    const int32_t n = st->n;
    const RowDesc dp = load_desc(&st->dp), dq = load_desc(&st->dq);
    const uint64_t *mass = a.tile_mass + (size_t)b * a.ntiles;
    static_assert(kTile / kSubTiles <= kWave, "a subtile fits one wave");
    DT x;
    draw_tile_params<DTT, DTD, NT>(x, a, b, n, dp, dq);
    const float u_s = a.u_s[b];
    // S and the tile holding floor(u * S): one round of loads when the tiles
    // fit one per thread (else a first sweep for S, a second for the pick)
    uint64_t S = 0;
    const int32_t rounds = (a.ntiles + NT - 1) / NT;
    uint64_t mk0 = 0;
    int32_t jr0 = 0, jr1 = 0;
    for (int32_t r = 0; r < rounds; ++r) {
        const int32_t kk = r * NT + (int32_t)threadIdx.x;
        const uint64_t mk = kk < a.ntiles ? mass[kk] : 0;
        if (r == 0) {
            mk0 = mk;
            if (a.d2t && kk < a.ntiles) {
                jr0 = min(max(a.tile_jb[kk], 0), a.Vd);
                jr1 = min(max(a.tile_jb[kk + 1], jr0), a.Vd);
            }
        }
        const uint64_t t = wave_total_u64(mk);
        if (lane == 0) s_tmp[wv] = t;
        __syncthreads();
        for (int w = 0; w < NW; ++w) S += s_tmp[w];
        __syncthreads();
    }
    int32_t tok = -1;
    if (S > 0) {
        const uint64_t target = frac_floor(u_s, S);    // < S
        if (threadIdx.x == 0) s_pick[0] = ~0ull;
        uint64_t run = 0;
        for (int32_t r = 0; r < rounds; ++r) {
            const int32_t kk = r * NT + (int32_t)threadIdx.x;
            const uint64_t mk = r == 0 ? mk0 : (kk < a.ntiles ? mass[kk] : 0);
            const uint64_t inc = wave_incl_scan_u64_dpp(mk);
            if (lane == kWave - 1) s_tmp[wv] = inc;
            __syncthreads();
            uint64_t base = run, tot = 0;
            for (int w = 0; w < NW; ++w) {
                if (w < wv) base += s_tmp[w];
                tot += s_tmp[w];
            }
            const uint64_t ex = base + inc - mk;
            if (kk < a.ntiles && mk > 0 && ex <= target && target < ex + mk) {
                s_pick[0] = (uint64_t)kk;                 // the bracket is unique
                s_pick[1] = target - ex;
                if (a.d2t) {
                    if (r > 0) {
                        jr0 = min(max(a.tile_jb[kk], 0), a.Vd);
                        jr1 = min(max(a.tile_jb[kk + 1], jr0), a.Vd);
                    }
                    s_jr[0] = jr0;
                    s_jr[1] = jr1;
                }
            }
            run += tot;
            __syncthreads();
        }
        if (s_pick[0] < (uint64_t)a.ntiles) {
            const int32_t kp = (int32_t)s_pick[0];
            const uint64_t tin = s_pick[1];
            const int32_t pj0 = a.d2t ? s_jr[0] : 0, pj1 = a.d2t ? s_jr[1] : 0;
            // one round of loads: the tile's subtile masses and, with d2t, the
            // target ids of its draft ids
            const int32_t sw = a.tile / kSubTiles, t0 = kp * a.tile;
            uint64_t sm = 0;
            if (wv == 0) sm = a.tile_sub[((size_t)b * a.ntiles + kp) * kSubTiles + lane];
            constexpr int UJ = kTile / NT;
            int32_t tj[UJ];
            const bool mapped = x.mapped && pj1 > pj0;
            if (mapped) {
#pragma unroll
                for (int u = 0; u < UJ; ++u) tj[u] = a.d2t[min(pj0 + u * NT + (int32_t)threadIdx.x, pj1 - 1)];
            }
            if ((int32_t)threadIdx.x < sw) s_qj[threadIdx.x] = -1;
            if (threadIdx.x == 0) {
                s_sp[0] = 0;
                s_sp[1] = ~0ull;                          // no token unless a subtile brackets tin
            }
            if (wv == 0) {
                // the subtile holding tin (exact sums, so the bracket is unique)
                const uint64_t inc = wave_incl_scan_u64_dpp(sm);
                if (sm > 0 && inc - sm <= tin && tin < inc) {
                    s_sp[0] = (uint64_t)lane;
                    s_sp[1] = tin - (inc - sm);
                }
            }
            __syncthreads();
            const int32_t ts = t0 + (int32_t)s_sp[0] * sw;
            const uint64_t tin2 = s_sp[1];
            if (mapped) {
#pragma unroll
                for (int u = 0; u < UJ; ++u) {
                    const int32_t j = pj0 + u * NT + (int32_t)threadIdx.x;
                    const int32_t ii = tj[u] - ts;
                    if (j < pj1 && ii >= 0 && ii < sw) s_qj[ii] = j;
                }
            }
            if (threadIdx.x == 0) s_tok = -1;
            __syncthreads();
            if (wv == 0) {
                // one wave weighs the subtile's ids in order, as the tile pass did
                const int32_t t = ts + lane;
                const bool v = lane < sw && t < a.Vt;
                const float zt = Elem<DTT>::load(x.trow, min(t, a.Vt - 1));
                float q = 0.0f;
                if (x.resid) {
                    const int32_t j = x.mapped ? (lane < sw ? s_qj[lane] : -1) : min(t, a.Vd - 1);
                    const float zq = Elem<DTD>::load(x.drow, max(j, 0));
                    if (j >= 0) q = x.qprob(zq);
                }
                const uint64_t w = v ? x.weight_q(zt, q) : 0ull;
                const uint64_t inc = wave_incl_scan_u64_dpp(w);
                const uint64_t hb = __ballot(w > 0 && inc > tin2 && inc - w <= tin2);
                // The weights are those the tile pass summed (same helpers, no
                // contraction), so one id brackets tin2; should none, the
                // subtile's last id of positive weight is drawn, the rule for
                // a draw that rounding leaves without a crossing.
                const uint64_t pb = __ballot(w > 0);
                if (lane == 0 && (hb || pb))
                    s_tok = hb ? ts + __ffsll((unsigned long long)hb) - 1 : ts + 63 - __clzll((long long)pb);
            }
            __syncthreads();
            tok = s_tok;
        }
    } else if (n < g) {
        // zero residual mass (p == q wherever p > 0): draw from p_n itself
        DrawCtx y;
        y.trow = reinterpret_cast<const char *>(a.tl) + ((size_t)b * (g + 1) + n) * (size_t)a.Vt * Elem<DTT>::kBytes;
        y.drow = reinterpret_cast<const char *>(a.dl) + ((size_t)b * g + n) * (size_t)a.Vd * Elem<DTD>::kBytes;
        y.d2t = nullptr;
        y.Vd = a.Vd;
        y.dp = dp;
        y.dq = y.dp;
        y.c = a.c;
        y.resid = false;
        tok = draw_row_one_wg<DTT, DTD, NT>(y, a.Vt, a.tile, (double)u_s, s_q, s_dtmp, s_itmp, s_j);
    }
    if (threadIdx.x == 0) a.out_tokens[(size_t)b * (g + 1) + n] = tok;
}


// ---------------------------------------------------------------------------
// Host side: workspace layout and launches
// ---------------------------------------------------------------------------


template <int DTT, int DTD>
static hipError_t launch_sample_dt(const SampleArgs &a, hipStream_t st) {
    const int32_t NR = 2 * a.gamma + 1;
    if (a.topp) {
        hipLaunchKernelGGL((topp_kernel<DTT, DTD, kToppThreads, kToppUnroll>), dim3(a.B * NR), dim3(kToppThreads), 0,
                           st, a);
        return hipGetLastError();
    }
    const int64_t per_seq = (int64_t)(a.gamma + 1) * a.Ct + (int64_t)a.gamma * a.Cd;
    hipLaunchKernelGGL((stats_kernel<DTT, DTD, kStatsThreads, kStatsUnroll>), dim3((unsigned)(a.B * (1 + per_seq))),
                       dim3(kStatsThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tile_kernel<DTT, DTD, kSampThreads>), dim3((unsigned)(a.B * a.ntiles)), dim3(kSampThreads),
                       sizeof(RowDesc) * (size_t)NR, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pick_kernel<DTT, DTD, kSampThreads>), dim3((unsigned)a.B), dim3(kSampThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs &a, int dt_t, int dt_d, hipStream_t st) {
    if (dt_t == SV_BF16 && dt_d == SV_BF16) return launch_sample_dt<SV_BF16, SV_BF16>(a, st);
    if (dt_t == SV_BF16 && dt_d == SV_F32) return launch_sample_dt<SV_BF16, SV_F32>(a, st);
    if (dt_t == SV_F32 && dt_d == SV_BF16) return launch_sample_dt<SV_F32, SV_BF16>(a, st);
    return launch_sample_dt<SV_F32, SV_F32>(a, st);
}

}  // namespace sv
