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
// One launch.  Each row is cut into C contiguous chunks; one workgroup streams
// one chunk once from HBM (16-byte loads, U vectors in flight per lane) and
// keeps a per-lane (max, lowest index).  The chunk's argmax goes to the
// workspace; the last workgroup of a sequence to arrive (atomic counter)
// combines the chunks of every row in chunk order and runs the walk.  No host
// synchronization; the time is the HBM read.
#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void greedy_kernel(GreedyArgs a) {
    __shared__ ArgMax red[NT / kWave];
    __shared__ int last_flag;
    __shared__ int32_t s_n, s_status;
    // epilogue scratch, sized by the launch: gmax[R] int32, then (tree) depth[R] int16, acc[R] uint8
    extern __shared__ int32_t gmax[];

    const int32_t R = a.rows_per_seq, C = a.chunks;
    const int32_t wg = blockIdx.x;
    const int32_t c = wg % C;
    const int32_t row = wg / C;           // b * R + r
    const int32_t b = row / R;

    // ---- stream one chunk of one row -----------------------------------
    const void *rowp = reinterpret_cast<const char *>(a.logits) +
                       (size_t)row * (size_t)a.V * Elem<DT>::kBytes;
    const RowSplit s = row_split<DT>(rowp, a.V);
    const int32_t lo = (int32_t)(((int64_t)s.nvec * c) / C);
    const int32_t hi = (int32_t)(((int64_t)s.nvec * (c + 1)) / C);
    ArgMax best;
    best.v = -INFINITY;
    best.i = INT32_MAX;
    stream_row<DT, U, NT>(rowp, s, lo, hi, c == 0, c == C - 1, [&](float v, int32_t i) {
        // indices rise per lane, so a strict '>' keeps the lowest index
        if (v > best.v) { best.v = v; best.i = i; }
    });
    best = wave_argmax(best);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgMax r0 = red[0];
        for (int w = 1; w < NT / kWave; ++w) r0 = argmax_merge(r0, red[w]);
        a.part[(size_t)row * C + c] = r0;
    }

    // ---- last workgroup of the sequence: combine and walk ----------------
    if (!arrive_last(&a.counters[b], (uint32_t)(R * C), &last_flag)) return;

    if (threadIdx.x == 0) { s_status = 0; s_n = 0; }
    __syncthreads();
    for (int32_t r = threadIdx.x; r < R; r += NT) {
        const ArgMax *p = a.part + ((size_t)b * R + r) * C;
        ArgMax m = p[0];
        for (int32_t k = 1; k < C; ++k) m = argmax_merge(m, p[k]);
        // a row of -inf everywhere: the lowest id attaining the maximum is 0
        if (m.i == INT32_MAX) m.i = 0;
        if (!(m.v > -INFINITY) || m.v == INFINITY) atomicOr(&s_status, (int)SV_SEQ_NO_MASS);
        gmax[r] = m.i;
    }
    __syncthreads();

    if (!a.tree) {
        // chain: x_i are the draft tokens, i < gamma = R - 1
        const int32_t g = R - 1;
        const int32_t *x = a.tokens + (size_t)b * g;
        if (threadIdx.x == 0) {
            int32_t n = g;
            for (int32_t i = 0; i < g; ++i)
                if (x[i] != gmax[i]) { n = i; break; }
            s_n = n;
        }
        for (int32_t i = threadIdx.x; i < g; i += NT)
            if (x[i] < 0 || x[i] >= a.V) atomicOr(&s_status, (int)SV_SEQ_TOKEN_RANGE);
        __syncthreads();
        const int32_t n = s_n;
        for (int32_t i = threadIdx.x; i <= g; i += NT)
            a.out_tokens[(size_t)b * (g + 1) + i] = i < n ? x[i] : (i == n ? gmax[n] : -1);
        if (threadIdx.x == 0) {
            a.out_len[b] = n;
            if (a.out_status) a.out_status[b] = s_status;
        }
        return;
    }

    // tree: node k >= 1 has parent par[k] < k and token tok[k]
    const int32_t N = R;
    const int32_t *tok = a.tokens + (size_t)b * N;
    const int32_t *par = a.parents + (size_t)b * N;
    int16_t *depth = reinterpret_cast<int16_t *>(gmax + N);
    uint8_t *acc = reinterpret_cast<uint8_t *>(depth + N);
    for (int32_t k = 1 + threadIdx.x; k < N; k += NT) {
        if (tok[k] < 0 || tok[k] >= a.V) atomicOr(&s_status, (int)SV_SEQ_TOKEN_RANGE);
        if (par[k] < 0 || par[k] >= k) atomicOr(&s_status, (int)SV_SEQ_BAD_PARENT);
    }
    if (threadIdx.x == 0) {
        // parents precede children, so one pass in index order settles every node
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
    const size_t lds = R * sizeof(int32_t) + (a.tree ? R * (sizeof(int16_t) + sizeof(uint8_t)) : 0);
    hipLaunchKernelGGL((greedy_kernel<DT, kGreedyThreads, kGreedyUnroll>), dim3(grid),
                       dim3(kGreedyThreads), lds, st, a);
    return hipGetLastError();
}

// Chunks per row.  Counted in 8-element vectors whatever the dtype, so the
// workspace size depends on V only (a float32 chunk is twice the bytes).
int32_t greedy_chunks(int32_t V, int /*dtype*/) {
    const int64_t nvec = ((int64_t)V + 7) / 8;
    const int64_t target = (int64_t)kGreedyThreads * kGreedyUnroll * kGreedyItersPerWg;
    int64_t C = (nvec + target - 1) / target;
    if (C < 1) C = 1;
    if (C > kMaxChunks) C = kMaxChunks;
    return (int32_t)C;
}

hipError_t launch_greedy(const GreedyArgs &a, int dtype, hipStream_t st) {
    const int64_t grid = (int64_t)a.B * a.rows_per_seq * a.chunks;
    if (dtype == SV_BF16) return launch_greedy_dt<SV_BF16>(a, (int)grid, st);
    return launch_greedy_dt<SV_F32>(a, (int)grid, st);
}

}  // namespace sv
