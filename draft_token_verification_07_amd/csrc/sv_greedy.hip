// sv_greedy.hip -- greedy (temperature-0) chain and tree verification.
//
// Greedy verification (SSD inference-engine guide, sec. 7, temperature-0
// runs; the 2.16x EAGLE blog's table asks for output identical to the
// target's own greedy decoding) needs the argmax of every target row, then a
// short sequential walk per sequence:
//   chain: n = first i with x_i != argmax(row i), emit x_0..x_{n-1}, argmax(row n);
//   tree (EAGLE blog sec. 5): node k is accepted iff its parent is and its token
//   is the argmax of the parent's row; the deepest accepted node wins (lowest
//   index on ties); emit the root->winner path and the winner row's argmax.
//
// Each row is cut into C contiguous chunks; one workgroup streams one chunk
// once from HBM (16-byte loads, U vectors in flight per lane) and keeps a
// per-lane (max, lowest index).  Short chains of whole rows finish in one
// launch: the last row of a sequence to arrive (atomic counter) combines the
// row results and takes the first mismatch.  Trees, long chains and chunked
// rows end the launch after the chunk results; a second launch with one
// workgroup per sequence merges the chunks in chunk order and runs the chain
// or the walk.  No host synchronization; the time is the HBM read.
#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

template <int NT>
__device__ __forceinline__ void greedy_sequence(const GreedyArgs &a, int32_t b, int32_t *gmax);

// SPLIT: the launch ends after the row (or chunk) results; seq_kernel merges
// the chunks of each row and runs the combine and walk.  Taken for sequences
// of more than kRowGroup rows and for rows cut in chunks (a kernel boundary
// costs less than the arrival levels it replaces).
template <int DT, int NT, int U, bool SPLIT>
__global__ __launch_bounds__(NT) void greedy_kernel(GreedyArgs a) {
    __shared__ ArgMax red[NT / kWave];
    __shared__ int last_flag;
    // epilogue scratch, sized by the launch: gmax[R], tok[R] int32, then
    // (tree) par[R] int32, depth[R] int16, acc[R] uint8
    extern __shared__ int32_t gmax[];

    const int32_t R = a.rows_per_seq, C = a.chunks;
    const int32_t wg = blockIdx.x;
    const int32_t c = wg % C;
    const int32_t row = wg / C;           // b * R + r
    const int32_t b = row / R;

    // ---- stream one chunk of one row -----------------------------------
    // Per lane: the running maximum over each iteration's U vectors costs one
    // max3 per two elements; the index is recovered only when a lane's
    // maximum improves (rare after the first iterations).  Indices rise per
    // lane, so a strict '>' keeps the lowest index among equal values.
    using E = Elem<DT>;
    const void *rowp = reinterpret_cast<const char *>(a.logits) +
                       (size_t)row * (size_t)a.V * E::kBytes;
    const RowSplit s = row_split<DT>(rowp, a.V);
    const int32_t lo = (int32_t)(((int64_t)s.nvec * c) / C);
    const int32_t hi = (int32_t)(((int64_t)s.nvec * (c + 1)) / C);
    ArgMax best;
    best.v = -INFINITY;
    best.i = INT32_MAX;
    auto one = [&](float v, int32_t i) {
        if (v > best.v) { best.v = v; best.i = i; }
    };
    const int tid = threadIdx.x;
    if (c == 0 && tid < s.head) one(E::load(rowp, tid), tid);
    const u32x4 *body = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(rowp) +
                                                        (size_t)s.head * E::kBytes);
    int32_t v = lo + tid;
    // U vectors per lane per round, all loaded before any is used.  Loads
    // are unconditional: in the last round they are clamped to the chunk's
    // last vector and the repeats are masked to -inf (a load under a
    // divergent branch would be waited for inside it, one round trip each).
    for (; v < hi; v += U * NT) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = __builtin_nontemporal_load(&body[min(v + u * NT, hi - 1)]);
        float x[U][E::kPerVec];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            E::unpack(raw[u], x[u]);
            if (v + u * NT >= hi) {
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) x[u][k] = -INFINITY;
            }
        }
        float tm = x[0][0];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) tm = fmaxf(tm, x[u][k]);
        if (tm > best.v) {
            int32_t idx = INT32_MAX;
#pragma unroll
            for (int u = U - 1; u >= 0; --u)
#pragma unroll
                for (int k = E::kPerVec - 1; k >= 0; --k)
                    if (x[u][k] == tm) idx = s.head + (v + u * NT) * E::kPerVec + k;
            best.v = tm;
            best.i = idx;
        }
    }
    if (c == C - 1 && tid < s.tail) {
        const int32_t i = s.head + s.nvec * E::kPerVec + tid;
        one(E::load(rowp, i), i);
    }
    best = wave_argmax(best);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = best;
    __syncthreads();
    ArgMax r0 = red[0];
    for (int w = 1; w < NT / kWave; ++w) r0 = argmax_merge(r0, red[w]);

    if constexpr (SPLIT) {
        // the sequence launch merges the chunks of each row
        if (threadIdx.x == 0) {
            if (C > 1) pub(&a.part[(size_t)row * C + c], r0);
            else pub(&a.rowres[row], r0);
        }
        return;
    }
    // (not split: the rows are whole, C == 1)
    if (threadIdx.x == 0) pub(&a.rowres[row], r0);

    // ---- last workgroup of the sequence: combine and walk ----------------
    if (!arrive_last(&a.counters[b], (uint32_t)R, &last_flag)) return;
    greedy_sequence<NT>(a, b, gmax);
}

// One workgroup per sequence, after greedy_kernel<..., true>.
template <int NT>
__global__ __launch_bounds__(NT) void seq_kernel(GreedyArgs a) {
    extern __shared__ int32_t gmax[];
    greedy_sequence<NT>(a, blockIdx.x, gmax);
}

// Combine the row results of sequence b and run the chain or the tree walk.
template <int NT>
__device__ __forceinline__ void greedy_sequence(const GreedyArgs &a, int32_t b, int32_t *gmax) {
    __shared__ int32_t s_n, s_status;
    const int32_t R = a.rows_per_seq;
    // one round of loads: the row results, the draft tokens (and parents)
    static_assert(NT >= kWave, "one wave at least");
    const int32_t nt = a.tree ? R : R - 1;               // tokens per sequence
    if (threadIdx.x == 0) { s_status = 0; s_n = a.tree ? 0 : R - 1; }
    int32_t *tok = gmax + R;                              // [R] (tree and chain)
    int32_t *par = tok + R;                               // [R] (tree)
    for (int32_t r = threadIdx.x; r < R; r += NT) {
        ArgMax m;
        if (a.split_chunks) {
            // the row's chunk results, merged in chunk order
            const ArgMax *pr = a.part + ((size_t)b * R + r) * a.chunks;
            m = sub(&pr[0]);
            for (int32_t k = 1; k < a.chunks; ++k) m = argmax_merge(m, sub(&pr[k]));
        } else {
            m = sub(&a.rowres[(size_t)b * R + r]);
        }
        const int32_t t = r < nt ? a.tokens[(size_t)b * nt + r] : 0;
        const int32_t p = a.tree ? a.parents[(size_t)b * R + r] : 0;
        // a row of -inf everywhere: the lowest id attaining the maximum is 0
        gmax[r] = m.i == INT32_MAX ? 0 : m.i;
        tok[r] = t;
        if (a.tree) par[r] = p;
        if (!(m.v > -INFINITY) || m.v == INFINITY) atomicOr(&s_status, (int)SV_SEQ_NO_MASS);
        const bool tok_used = a.tree ? r >= 1 : r < nt;
        if (tok_used && (t < 0 || t >= a.V)) atomicOr(&s_status, (int)SV_SEQ_TOKEN_RANGE);
        if (a.tree && r >= 1 && (p < 0 || p >= r)) atomicOr(&s_status, (int)SV_SEQ_BAD_PARENT);
    }
    __syncthreads();

    if (!a.tree) {
        // chain: x_i are the draft tokens, i < gamma = R - 1
        const int32_t g = R - 1;
        for (int32_t i = threadIdx.x; i < g; i += NT)
            if (tok[i] != gmax[i]) atomicMin(&s_n, i);        // first mismatch
        __syncthreads();
        const int32_t n = s_n;
        for (int32_t i = threadIdx.x; i <= g; i += NT)
            a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? tok[i] : (i == n ? gmax[n] : -1);
        if (threadIdx.x == 0) {
            a.out_len[b] = n;
            if (a.out_status) a.out_status[b] = s_status;
        }
        return;
    }

    // tree: node k >= 1 has parent par[k] < k and token tok[k].  Node k is
    // accepted iff every edge on its path to the root matches (the edge into
    // k matches when tok[k] is the argmax of the parent's row); a node with
    // a bad parent is accepted by no one below it.
    const int32_t N = R;
    int16_t *depth = reinterpret_cast<int16_t *>(par + N);
    if (N <= kWave) {
        // one wave, pointer jumping: after round r every node points 2^r
        // levels up (or at its root) and carries the AND of the edges and the
        // length of the path jumped so far
        if (threadIdx.x < kWave) {
            const int32_t k = threadIdx.x;
            const bool node = k < N;
            const int32_t p = node ? par[k] : 0;
            const bool root = k == 0 || !node || p < 0 || p >= k;
            int32_t up = root ? k : p;
            bool ok = root ? (k == 0) : tok[k] == gmax[p];
            int32_t dep = root ? 0 : 1;
            for (int r = 0; r < 6; ++r) {                  // 2^6 = 64 >= any depth here
                const int32_t up2 = __shfl(up, up, kWave);
                const bool ok2 = __shfl((int)ok, up, kWave) != 0;
                const int32_t dep2 = __shfl(dep, up, kWave);
                ok = ok && ok2;
                dep += dep2;
                up = up2;
            }
            // the deepest accepted node, lowest index on ties
            const int32_t key = (node && ok) ? (dep << 16) | (0xffff - k) : -1;
            const int32_t best = wave_max(key);
            if (node) depth[k] = (int16_t)dep;
            if (k == 0) s_n = best >= 0 ? 0xffff - (best & 0xffff) : 0;
        }
    } else if (threadIdx.x == 0) {
        // parents precede children, so one pass in index order settles every node
        uint8_t *acc = reinterpret_cast<uint8_t *>(depth + N);
        acc[0] = 1;
        depth[0] = 0;
        int32_t best_k = 0;
        for (int32_t k = 1; k < N; ++k) {
            const int32_t p = par[k];
            if (p < 0 || p >= k) { acc[k] = 0; depth[k] = 0; continue; }
            depth[k] = (int16_t)(depth[p] + 1);
            acc[k] = acc[p] && tok[k] == gmax[p];
            if (acc[k] && depth[k] > depth[best_k]) best_k = k;
        }
        s_n = best_k;
    }
    __syncthreads();
    const int32_t best_k = s_n;
    const int32_t d = depth[best_k];
    // the path, written from the winner back to the root's child
    if (threadIdx.x == 0) {
        int32_t node = best_k;
        for (int32_t sdx = d - 1; sdx >= 0; --sdx) {
            a.out_path[(size_t)b * N + sdx] = node;
            a.out_tokens[(size_t)b * N + sdx] = tok[node];
            node = par[node];
        }
        a.out_tokens[(size_t)b * N + d] = gmax[best_k];
        a.out_len[b] = d;
        if (a.out_status) a.out_status[b] = s_status;
    }
    for (int32_t k = threadIdx.x; k < N; k += NT) {
        if (k >= d) a.out_path[(size_t)b * N + k] = -1;
        if (k > d) a.out_tokens[(size_t)b * N + k] = -1;
    }
}

template <int DT>
static hipError_t launch_greedy_dt(const GreedyArgs &a, int grid, hipStream_t st) {
    const size_t R = (size_t)a.rows_per_seq;
    // gmax[R], tok[R], then (tree) par[R], depth[R] int16, acc[R] uint8
    const size_t lds = 2 * R * sizeof(int32_t) + (a.tree ? R * (sizeof(int32_t) + sizeof(int16_t) + sizeof(uint8_t)) : 0);
    if (!greedy_split(a.rows_per_seq, a.chunks)) {
        hipLaunchKernelGGL((greedy_kernel<DT, kGreedyThreads, kGreedyUnroll, false>), dim3(grid),
                           dim3(kGreedyThreads), lds, st, a);
        return hipGetLastError();
    }
    // Few workgroups (at most two per CU): twice the threads each, so that a
    // CU keeps as many loads in flight as with more rows
    if (grid <= kGreedyWideMaxWgs)
        hipLaunchKernelGGL((greedy_kernel<DT, SV_GREEDY_WIDE * kGreedyThreads, kGreedyUnroll, true>), dim3(grid),
                           dim3(SV_GREEDY_WIDE * kGreedyThreads), 0, st, a);
    else
        hipLaunchKernelGGL((greedy_kernel<DT, kGreedyThreads, kGreedyUnroll, true>), dim3(grid), dim3(kGreedyThreads),
                           0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((seq_kernel<kGreedyThreads>), dim3(a.B), dim3(kGreedyThreads), lds, st, a);
    return hipGetLastError();
}


// The sequence step alone, on row results already in a.rowres (one per row,
// published): the chain or the tree walk, one workgroup per sequence.
hipError_t launch_seq(const GreedyArgs &a, hipStream_t st) {
    const size_t R = (size_t)a.rows_per_seq;
    const size_t lds = 2 * R * sizeof(int32_t) + (a.tree ? R * (sizeof(int32_t) + sizeof(int16_t) + sizeof(uint8_t)) : 0);
    hipLaunchKernelGGL((seq_kernel<kGreedyThreads>), dim3(a.B), dim3(kGreedyThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_greedy(const GreedyArgs &a, int dtype, hipStream_t st) {
    const int64_t grid = (int64_t)a.B * a.rows_per_seq * a.chunks;
    if (dtype == SV_BF16) return launch_greedy_dt<SV_BF16>(a, (int)grid, st);
    return launch_greedy_dt<SV_F32>(a, (int)grid, st);
}

}  // namespace sv
