// sv_lmhead.hip -- the fused lm_head -> greedy verification.
//
// The target's logits over the gamma+1 verified positions are the product of
// the last hidden states and the lm_head weight (SSD inference-engine guide,
// sec. 6: compute_logits turns the hidden states into logits, and for the
// EAGLE3 draft head scatters them through d2t; the 2.16x EAGLE blog, sec. 6,
// ties the cost of this classification matmul to the vocabulary).  Greedy
// verification (SSD guide sec. 7, temperature 0) needs only the argmax of each
// row, so the logits are never written: each GEMM tile reduces its rows to a
// (logit, lowest id) maximum in its epilogue.
//
// logits[m][v] = sum_k hidden[m][k] * W[v][k], bfloat16 inputs, float32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16: per lane, A
// holds row l%16 and k 8(l/16)..+7, B column l%16 and the same k, and the
// 16x16 result rows 4(l/16)..+3 of column l%16).  A workgroup of four waves
// computes a 128 x 128 tile, each wave 64 x 64 (4 x 4 MFMA tiles), 32 k per
// step, with the next step's operands loaded before the current step's
// MFMAs.  Operands come straight from global memory as 16-byte loads (both
// matrices are k-contiguous).  The block order puts the row tiles that share
// a weight tile on one XCD, so the weights are read from HBM about once.
//
// Epilogue: per row and 128-column tile, the largest logit and its lowest id
// as one 64-bit key (order-preserving key of the value, then ~id), stored
// per tile.  lmhead_reduce_kernel takes the maximum key of each row and
// publishes the row result, and the sequence step (chain or tree walk) of
// the greedy path follows.
#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kLmThreads = 256;

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t *p, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4 *>(p);
    return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kLmThreads) void lmhead_kernel(LmheadArgs a) {
    __shared__ uint64_t s_key[kLmTile][2];
    // block -> (row tile, column tile): the row tiles of one column tile on one XCD
    const int32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int32_t mt = slot % a.mtiles;
    const int32_t nt = (slot / a.mtiles) * 8 + xcd;
    if (nt >= a.ntiles) return;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int wm = wv >> 1, wn = wv & 1;
    const int32_t m0 = mt * kLmTile + wm * 64, n0 = nt * kLmTile + wn * 64;
    const int lr = lane & 15, lk = (lane >> 4) * 8;
    const int32_t d = a.d;
    // operand rows of this lane (clamped; rows past M or V are masked in the epilogue)
    const uint16_t *ap[4], *bp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t r = min(m0 + 16 * i + lr, a.M - 1);
        const int32_t c = min(n0 + 16 * i + lr, a.V - 1);
        ap[i] = a.hidden + (size_t)r * d + lk;
        bp[i] = a.W + (size_t)c * d + lk;
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = ld_frag(ap[i], lk < d);
        fb[i] = ld_frag(bp[i], lk < d);
    }
    for (int32_t k0 = 0; k0 < d; k0 += 32) {
        // the next step's operands first (zero past d)
        const bool nok = k0 + 32 + lk < d;
        bf16x8 na[4], nb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            na[i] = ld_frag(ap[i] + k0 + 32, nok);
            nb[i] = ld_frag(bp[i] + k0 + 32, nok);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = na[i];
            fb[i] = nb[i];
        }
    }
    // epilogue: per row, the largest logit over this wave's 64 columns, lowest
    // id on ties -- per lane over its four columns, then over the 16 lanes of
    // the lane group holding the same rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int32_t r = m0 + 16 * i + (lane >> 4) * 4 + e;
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int32_t c = n0 + 16 * j + lr;
                const uint64_t key = c < a.V ? (((uint64_t)zkey(acc[i][j][e]) << 32) | (uint32_t)~(uint32_t)c) : 0ull;
                best = key > best ? key : best;
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                                       (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
                best = other > best ? other : best;
            }
            if (lr == 0) s_key[wm * 64 + 16 * i + (lane >> 4) * 4 + e][wn] = best;
            (void)r;
        }
    }
    __syncthreads();
    if (threadIdx.x < kLmTile) {
        const int32_t r = mt * kLmTile + (int32_t)threadIdx.x;
        const uint64_t k0 = s_key[threadIdx.x][0], k1 = s_key[threadIdx.x][1];
        if (r < a.M) a.part[(size_t)r * a.ntiles + nt] = k0 > k1 ? k0 : k1;
    }
}

// One wave per row: the maximum key over the row's column tiles, published
// as the row result (value, id); optionally written out.
__global__ __launch_bounds__(256) void lmhead_reduce_kernel(LmheadArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t r = blockIdx.x * 4 + (int32_t)(threadIdx.x / kWave);
    if (r >= a.M) return;
    const uint64_t *p = a.part + (size_t)r * a.ntiles;
    uint64_t best = 0;
    for (int32_t c = lane; c < a.ntiles; c += kWave) best = p[c] > best ? p[c] : best;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                               (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
        best = other > best ? other : best;
    }
    if (lane == 0) {
        ArgMax m;
        m.v = fkey_inv((uint32_t)(best >> 32));
        m.i = (int32_t)~(uint32_t)best;
        pub(&a.rowres[r], m);
        if (a.out_argmax) a.out_argmax[r] = m.i;
        if (a.out_maxlogit) a.out_maxlogit[r] = m.v;
    }
}

hipError_t launch_lmhead(const LmheadArgs &a, hipStream_t st) {
    const int64_t grid = (int64_t)a.mtiles * a.ntiles8;
    hipLaunchKernelGGL(lmhead_kernel, dim3((unsigned)grid), dim3(kLmThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_reduce_kernel, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
