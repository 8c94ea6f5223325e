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
// computes a 128 x 256 tile, each wave 64 x 128 (4 x 8 MFMA tiles), 32 k per
// step.  Both matrices are k-contiguous: each step's operands are read as
// coalesced 16-byte loads into registers while the matrix cores work on the
// previous step, then written to the other half of a double-buffered LDS
// stage (rows padded by 16 bytes), from which the waves take their MFMA
// fragments.  The block order puts the row tiles that share
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
constexpr int kLmBM = 128;                 // rows per workgroup tile
constexpr int kLmBN = kLmTile * 2;         // columns per workgroup tile (two key tiles)
constexpr int kLmBK = 32;                  // k per stage (one MFMA k)
constexpr int kLmPitch = kLmBK * 2 + 16;   // LDS bytes per operand row (64 + 16 of padding)

// One k-step of both operands in registers: A [kLmBM rows][64 B] and
// B [kLmBN rows][64 B]; thread t holds the 16-byte pieces t, t + 256, ... of
// the row-major [row][4 pieces] order (four threads per row, coalesced).
struct Stage {
    u32x4 a[kLmBM * 4 / kLmThreads];
    u32x4 b[kLmBN * 4 / kLmThreads];
};

__device__ __forceinline__ void stage_load(Stage &st, const uint16_t *A, const uint16_t *B, int32_t m0, int32_t n0,
                                           int32_t M, int32_t V, int32_t d, int32_t k0) {
#pragma unroll
    for (int u = 0; u < kLmBM * 4 / kLmThreads; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        const int32_t r = min(m0 + p / 4, M - 1);
        const int32_t k = k0 + (p % 4) * 8;
        st.a[u] = k < d ? *reinterpret_cast<const u32x4 *>(A + (size_t)r * d + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLmBN * 4 / kLmThreads; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        const int32_t c = min(n0 + p / 4, V - 1);
        const int32_t k = k0 + (p % 4) * 8;
        st.b[u] = k < d ? *reinterpret_cast<const u32x4 *>(B + (size_t)c * d + k) : u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void stage_store(const Stage &st, unsigned char *sa, unsigned char *sb) {
#pragma unroll
    for (int u = 0; u < kLmBM * 4 / kLmThreads; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        *reinterpret_cast<u32x4 *>(sa + (p / 4) * kLmPitch + (p % 4) * 16) = st.a[u];
    }
#pragma unroll
    for (int u = 0; u < kLmBN * 4 / kLmThreads; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        *reinterpret_cast<u32x4 *>(sb + (p / 4) * kLmPitch + (p % 4) * 16) = st.b[u];
    }
}

__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_kernel(LmheadArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][kLmBM * kLmPitch];
    __shared__ __attribute__((aligned(16))) unsigned char s_b[2][kLmBN * kLmPitch];
    __shared__ uint64_t s_key[kLmBM][2];
    // block -> (row tile, column tile): the row tiles of one column tile on one XCD
    const int32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int32_t mt = slot % a.mtiles;
    const int32_t nt2 = (slot / a.mtiles) * 8 + xcd;            // 256-column tile
    if (nt2 * kLmBN >= a.V) return;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int wm = wv >> 1, wn = wv & 1;                         // wave tile: 64 rows x 128 columns
    const int32_t M = a.M, V = a.V, d = a.d;
    const int32_t bm0 = mt * kLmBM, bn0 = nt2 * kLmBN;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Stage st;
    stage_load(st, a.hidden, a.W, bm0, bn0, M, V, d, 0);
    stage_store(st, s_a[0], s_b[0]);
    __syncthreads();
    int buf = 0;
    for (int32_t k0 = 0; k0 < d; k0 += kLmBK) {
        const bool more = k0 + kLmBK < d;
        if (more) stage_load(st, a.hidden, a.W, bm0, bn0, M, V, d, k0 + kLmBK);   // next stage, in flight
        const unsigned char *sa = s_a[buf] + (wm * 64 + lr) * kLmPitch + lg * 16;
        const unsigned char *sb = s_b[buf] + (wn * 128 + lr) * kLmPitch + lg * 16;
        bf16x8 fa[4], fb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sa + i * 16 * kLmPitch));
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sb + j * 16 * kLmPitch));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if (more) {
            // the buffer written here was last read before the previous barrier
            stage_store(st, s_a[buf ^ 1], s_b[buf ^ 1]);
            __syncthreads();
            buf ^= 1;
        }
    }
    // epilogue: per row, the largest logit over this wave's 128 columns (one
    // key tile), lowest id on ties -- per lane over its eight columns, then
    // over the 16 lanes of the lane group holding the same rows
    const int32_t n0 = bn0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t c = n0 + 16 * j + lr;
                const uint64_t key = c < V ? (((uint64_t)zkey(acc[i][j][e]) << 32) | (uint32_t)~(uint32_t)c) : 0ull;
                best = key > best ? key : best;
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                                       (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
                best = other > best ? other : best;
            }
            if (lr == 0) s_key[wm * 64 + 16 * i + lg * 4 + e][wn] = best;
        }
    }
    __syncthreads();
    {
        const int rr = threadIdx.x >> 1, half = threadIdx.x & 1;   // 256 threads: 128 rows x 2 key tiles
        const int32_t r = bm0 + rr;
        const int32_t nt = nt2 * 2 + half;
        if (r < M && nt < a.ntiles) a.part[(size_t)r * a.ntiles + nt] = s_key[rr][half];
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
