// sv_fanout.hip -- the SSD fan-out lookup.
//
// SSD inference-engine guide (lpnh.cn), sec. 1: while the target verifies,
// the draft pre-speculates the possible verification outcomes and drafts
// every branch at once, so a branch that matches the outcome makes the next
// round's drafting free; sec. 7 runs it with a fan-out of 3 (--f 3).  An
// outcome is (n, t): the accepted length and the token emitted after the
// accepted drafts, out_tokens[b, n].  For every n in [0, gamma] the caller's
// table holds f candidate tokens cand[b, n, j]; branch n * f + j carries L
// pre-drafted tokens.  The lookup returns the branch of the lowest slot whose
// candidate equals t (-1 when none does) and gathers its drafts.
//
// One wave per sequence: lane j tests slot j (f <= 64), a ballot gives the
// lowest matching slot, and the lanes copy the branch's drafts, coalesced.
#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

template <int NT>
__global__ __launch_bounds__(NT) void fanout_kernel(FanoutArgs a) {
    constexpr int NW = NT / kWave;
    __shared__ uint32_t s_hits;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int64_t b = (int64_t)blockIdx.x * NW + wv;
    if (threadIdx.x == 0) s_hits = 0;
    __syncthreads();
    const int32_t g1 = a.gamma + 1;
    if (b < a.B) {
        const int32_t n = a.accept_len[b];
        const bool ok = n >= 0 && n <= a.gamma;
        const int32_t t = ok ? a.out_tokens[b * g1 + n] : -1;
        const int32_t cnd = (ok && lane < a.f) ? a.cand[(b * g1 + n) * a.f + lane] : -1;
        const uint64_t m = __ballot(ok && lane < a.f && cnd >= 0 && cnd == t);
        const int32_t br = m ? n * a.f + (__ffsll((unsigned long long)m) - 1) : -1;
        if (lane == 0) {
            a.out_branch[b] = br;
            if (br >= 0) atomicAdd(&s_hits, 1u);
        }
        if (a.out_next) {
            const int32_t *src = a.drafts + ((b * g1 * a.f) + (br >= 0 ? br : 0)) * (int64_t)a.L;
            for (int32_t i = lane; i < a.L; i += kWave) a.out_next[b * a.L + i] = br >= 0 ? src[i] : -1;
        }
    }
    __syncthreads();
    if (a.counters && threadIdx.x == 0) {
        const int64_t first = (int64_t)blockIdx.x * NW;
        const int64_t nseq = a.B - first < NW ? a.B - first : NW;
        atomicAdd(&a.counters[0], (unsigned long long)nseq);
        if (s_hits) atomicAdd(&a.counters[1], (unsigned long long)s_hits);
    }
}

hipError_t launch_fanout(const FanoutArgs &a, hipStream_t st) {
    constexpr int NT = 256;
    const int64_t grid = (a.B + NT / kWave - 1) / (NT / kWave);
    hipLaunchKernelGGL((fanout_kernel<NT>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
