// sv_api.hip -- the launching entry points of the C ABI of libspecverify:
// each runs its argument check (sv_host.cpp), fills the argument block and
// dispatches the launches.  No allocation, no synchronization: every launch
// goes to the caller's stream, and host-detectable argument errors return
// before anything is launched.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sv_common.h"
#include "sv_internal.h"

using namespace sv;

// Scratch of the allocation-free entry point: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` is only a
// stand-in for the symbol; kernels receive the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Zero the counter region of the scratch array (a fill kernel rather than a
// memset, so that a caller capturing the stream records a kernel node).
__global__ void scratch_clear(u32x4 *p, size_t n) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

// The current device's scratch address, set up on the first call on that
// device: the symbol's address for this device, then its counter region
// cleared on `stream` (every call returns the counters to zero after that).
sv_status scratch_for_current_device(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SV_ERR_HIP;
    if (dev >= kMaxDevices) return SV_ERR_TOO_LARGE;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SV_ERR_HIP;
        const size_t n = counter_region(SV_NOALLOC_SCRATCH_BYTES) / sizeof(u32x4);
        hipLaunchKernelGGL(scratch_clear, dim3(256), dim3(256), 0, stream, static_cast<u32x4 *>(ptr), n);
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

namespace {

sv_status run_greedy(const void *logits, sv_dtype dt, const int32_t *tokens, const int32_t *parents,
                     int32_t B, int32_t R, int32_t V, bool tree, int32_t *out_tokens, int32_t *out_len,
                     int32_t *out_status, int32_t *out_path, void *ws, size_t ws_bytes, hipStream_t st) {
    GreedyArgs a;
    a.logits = logits;
    a.tokens = tokens;
    a.parents = parents;
    a.B = B;
    a.rows_per_seq = R;
    a.V = V;
    a.chunks = greedy_C(B, R, V);
    a.tree = tree ? 1 : 0;
    a.split_chunks = greedy_split(R, a.chunks) && a.chunks > 1 ? 1 : 0;
    a.out_tokens = out_tokens;
    a.out_len = out_len;
    a.out_status = out_status;
    a.out_path = out_path;
    char *base = static_cast<char *>(ws);
    char *data = base + counter_region(ws_bytes);
    a.counters = reinterpret_cast<uint32_t *>(base);
    a.rowres = reinterpret_cast<ArgMax *>(data);
    a.part = reinterpret_cast<ArgMax *>(data + greedy_rowres_bytes(B, R));
    return launch_greedy(a, dt, st) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status run_lmhead(const void *hidden, const void *W, const int32_t *tokens, const int32_t *parents, int32_t B,
                     int32_t R, int32_t d, int32_t V, bool tree, int32_t *out_path, int32_t *out_tokens,
                     int32_t *out_len, int32_t *out_argmax, float *out_maxlogit, int32_t *out_status, void *ws,
                     size_t ws_bytes, hipStream_t st) {
    const int64_t M = (int64_t)B * R;
    const size_t nt = ((size_t)V + kLmTile - 1) / kLmTile;
    LmheadArgs L;
    L.hidden = static_cast<const uint16_t *>(hidden);
    L.W = static_cast<const uint16_t *>(W);
    L.M = (int32_t)M;
    L.d = d;
    L.V = V;
    L.mtiles = (int32_t)((M + kLmTile - 1) / kLmTile);
    L.ntiles = (int32_t)nt;
    L.ntiles8 = (int32_t)lmhead_col_tiles8(V);
    char *data = static_cast<char *>(ws) + counter_region(ws_bytes);
    L.part = reinterpret_cast<uint64_t *>(data);
    L.rowres = reinterpret_cast<ArgMax *>(data + lmhead_part_bytes(M, V));
    L.out_argmax = out_argmax;
    L.out_maxlogit = out_maxlogit;
    if (launch_lmhead(L, st) != hipSuccess) return SV_ERR_HIP;
    GreedyArgs a;
    a.logits = nullptr;
    a.tokens = tokens;
    a.parents = parents;
    a.B = B;
    a.rows_per_seq = R;
    a.V = V;
    a.chunks = 1;
    a.tree = tree ? 1 : 0;
    a.split_chunks = 0;
    a.out_tokens = out_tokens;
    a.out_len = out_len;
    a.out_status = out_status;
    a.out_path = out_path;
    a.part = nullptr;
    a.rowres = L.rowres;
    a.counters = nullptr;
    return launch_seq(a, st) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" {

sv_status spec_verify_greedy(const void *target_logits, sv_dtype dtype, const int32_t *draft_tokens,
                             int32_t B, int32_t gamma, int32_t V, int32_t *out_tokens,
                             int32_t *out_accept_len, int32_t *out_status, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    bool go;
    const sv_status c = check_greedy(target_logits, dtype, draft_tokens, B, gamma, V, out_tokens, out_accept_len,
                                     workspace, workspace_bytes, &go);
    if (!go) return c;
    return run_greedy(target_logits, dtype, draft_tokens, nullptr, B, gamma + 1, V, false, out_tokens,
                      out_accept_len, out_status, nullptr, workspace, workspace_bytes, stream);
}

sv_status spec_verify_tree_greedy(const void *target_logits, sv_dtype dtype, const int32_t *node_tokens,
                                  const int32_t *parents, int32_t B, int32_t N, int32_t V,
                                  int32_t *out_path_nodes, int32_t *out_tokens, int32_t *out_accept_len,
                                  int32_t *out_status, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    bool go;
    const sv_status c = check_tree(target_logits, dtype, node_tokens, parents, B, N, V, out_path_nodes, out_tokens,
                                   out_accept_len, workspace, workspace_bytes, &go);
    if (!go) return c;
    return run_greedy(target_logits, dtype, node_tokens, parents, B, N, V, true, out_tokens, out_accept_len,
                      out_status, out_path_nodes, workspace, workspace_bytes, stream);
}

sv_status spec_verify_sample(const void *target_logits, sv_dtype target_dtype, const void *draft_logits,
                             sv_dtype draft_dtype, const int32_t *draft_tokens, const int32_t *d2t,
                             const float *u_accept, const float *u_sample, int32_t B, int32_t gamma,
                             int32_t Vt, int32_t Vd, float temperature, float top_p, int32_t *out_tokens,
                             int32_t *out_accept_len, float *out_p_tok, float *out_q_tok, int32_t *out_status,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    WorkspaceLayout L;
    int32_t Ct = 1, Cd = 1, tl = 1, nt = 1;
    bool go;
    const sv_status c = check_sample(target_logits, target_dtype, draft_logits, draft_dtype, draft_tokens, d2t,
                                     u_accept, u_sample, B, gamma, Vt, Vd, temperature, top_p, out_tokens,
                                     out_accept_len, workspace, workspace_bytes, &L, &Ct, &Cd, &tl, &nt, &go);
    if (!go) return c;
    SampleArgs a;
    a.tl = target_logits;
    a.dl = draft_logits;
    a.tokens = draft_tokens;
    a.d2t = d2t;
    a.u_acc = u_accept;
    a.u_s = u_sample;
    a.B = B;
    a.gamma = gamma;
    a.Vt = Vt;
    a.Vd = Vd;
    a.T = temperature;
    a.c = 1.4426950408889634f / temperature;     // log2(e) / T: 2^((z - m) c) = e^((z - m) / T)
    a.top_p = top_p;
    a.topp = top_p < 1.0f ? 1 : 0;
    a.Ct = Ct;
    a.Cd = Cd;
    a.tile = tl;
    a.ntiles = nt;
    a.out_tokens = out_tokens;
    a.out_len = out_accept_len;
    a.out_status = out_status;
    a.out_p = out_p_tok;
    a.out_q = out_q_tok;
    char *base = static_cast<char *>(workspace);
    char *data = base + counter_region(workspace_bytes);
    a.cnt_stats = reinterpret_cast<uint32_t *>(base + L.cnt_stats);
    a.map_flag = a.cnt_stats + B;
    a.seq = reinterpret_cast<SeqState *>(data + L.seq);
    a.rows = reinterpret_cast<RowDesc *>(data + L.rows);
    a.part = reinterpret_cast<MaxSum *>(data + L.part);
    a.kept = reinterpret_cast<KeptEnt *>(data + L.kept);
    a.kept_stride = kept_stride(Vt, Vd);
    a.probe = reinterpret_cast<Probe *>(data + L.probe);
    a.tile_mass = reinterpret_cast<uint64_t *>(data + L.tile_mass);
    a.tile_sub = reinterpret_cast<uint64_t *>(data + L.tile_sub);
    a.tile_jb = reinterpret_cast<int32_t *>(data + L.tile_jb);
    return launch_sample(a, target_dtype, draft_dtype, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_draft_sample(const void *logits, sv_dtype dtype, const int32_t *d2t, const float *u, int32_t B,
                            int32_t V, float temperature, float top_p, int32_t top_k, int32_t *out_tokens,
                            float *out_prob, int32_t *out_status, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    DraftLayout L;
    int32_t C = 1;
    bool go;
    const sv_status c = check_draft(logits, dtype, u, B, V, temperature, top_p, out_tokens, workspace,
                                    workspace_bytes, &L, &C, &go);
    if (!go) return c;
    DraftArgs a;
    a.logits = logits;
    a.d2t = d2t;
    a.u = u;
    a.B = B;
    a.V = V;
    a.C = C;
    a.T = temperature;
    a.c = 1.4426950408889634f / temperature;
    a.top_p = top_p;
    a.top_k = (top_k > 0 && top_k < V) ? top_k : 0;
    a.out_tokens = out_tokens;
    a.out_prob = out_prob;
    a.out_status = out_status;
    char *base = static_cast<char *>(workspace);
    char *data = base + counter_region(workspace_bytes);
    a.counters = reinterpret_cast<uint32_t *>(base);
    a.res = reinterpret_cast<ChunkRes *>(data + L.res);
    a.cand = reinterpret_cast<uint64_t *>(data + L.cand);
    a.desc = reinterpret_cast<RowDesc *>(data + L.desc);
    return launch_draft(a, dtype, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_verify_count(const int32_t *accept_len, int32_t B, int32_t gamma, uint64_t *counters,
                            hipStream_t stream) {
    bool go;
    const sv_status c = check_count(accept_len, B, gamma, counters, &go);
    if (!go) return c;
    return launch_count(accept_len, B, gamma, reinterpret_cast<unsigned long long *>(counters), stream) == hipSuccess
               ? SV_OK
               : SV_ERR_HIP;
}

sv_status spec_fanout_lookup(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                             const int32_t *branch_drafts, int32_t B, int32_t gamma, int32_t f, int32_t L,
                             int32_t *out_branch, int32_t *out_next, uint64_t *counters, hipStream_t stream) {
    bool go;
    const sv_status c = check_fanout(out_tokens, accept_len, cand, branch_drafts, B, gamma, f, L, out_branch,
                                     out_next, counters, &go);
    if (!go) return c;
    FanoutArgs a;
    a.out_tokens = out_tokens;
    a.accept_len = accept_len;
    a.cand = cand;
    a.drafts = branch_drafts;
    a.B = B;
    a.gamma = gamma;
    a.f = f;
    a.L = L;
    a.out_branch = out_branch;
    a.out_next = (L > 0) ? out_next : nullptr;
    a.counters = reinterpret_cast<unsigned long long *>(counters);
    return launch_fanout(a, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_vocab_trim(const int32_t *tokens, int64_t N, int32_t Vt, float P, int32_t *out_d2t,
                          int32_t *out_t2d, int32_t *out_vd, int64_t *out_info, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    bool go;
    const sv_status c = check_trim(tokens, N, Vt, P, out_d2t, out_vd, out_info, workspace, workspace_bytes, &go);
    if (!go) return c;
    TrimArgs a;
    a.tokens = tokens;
    a.N = N;
    a.Vt = Vt;
    a.P = P;
    a.out_d2t = out_d2t;
    a.out_t2d = out_t2d;
    a.out_vd = out_vd;
    a.out_info = out_info;
    char *base = static_cast<char *>(workspace);
    trim_layout(a, base, base + counter_region(workspace_bytes));
    return launch_trim(a, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_lmhead_verify_greedy(const void *hidden, const void *W, const int32_t *draft_tokens, int32_t B,
                                    int32_t gamma, int32_t d, int32_t V, int32_t *out_tokens, int32_t *out_accept_len,
                                    int32_t *out_argmax, float *out_maxlogit, int32_t *out_status, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    bool go;
    const sv_status c = check_lmhead(hidden, W, draft_tokens, nullptr, false, B, gamma + 1, d, V, nullptr, out_tokens,
                                     out_accept_len, workspace, workspace_bytes, &go);
    if (!go) return c;
    return run_lmhead(hidden, W, draft_tokens, nullptr, B, gamma + 1, d, V, false, nullptr, out_tokens,
                      out_accept_len, out_argmax, out_maxlogit, out_status, workspace, workspace_bytes, stream);
}

sv_status spec_lmhead_verify_tree(const void *hidden, const void *W, const int32_t *node_tokens,
                                  const int32_t *parents, int32_t B, int32_t N, int32_t d, int32_t V,
                                  int32_t *out_path_nodes, int32_t *out_tokens, int32_t *out_accept_len,
                                  int32_t *out_argmax, float *out_maxlogit, int32_t *out_status, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    bool go;
    const sv_status c = check_lmhead(hidden, W, node_tokens, parents, true, B, N, d, V, out_path_nodes, out_tokens,
                                     out_accept_len, workspace, workspace_bytes, &go);
    if (!go) return c;
    return run_lmhead(hidden, W, node_tokens, parents, B, N, d, V, true, out_path_nodes, out_tokens, out_accept_len,
                      out_argmax, out_maxlogit, out_status, workspace, workspace_bytes, stream);
}

sv_status spec_verify_sample_noalloc(const void *target_logits, sv_dtype target_dtype, const void *draft_logits,
                                     sv_dtype draft_dtype, const int32_t *draft_tokens, const int32_t *d2t,
                                     const float *u_accept, const float *u_sample, int32_t B, int32_t gamma,
                                     int32_t Vt, int32_t Vd, float temperature, float top_p, int32_t *out_tokens,
                                     int32_t *out_accept_len, float *out_p_tok, float *out_q_tok,
                                     int32_t *out_status, hipStream_t stream) {
    // sizes first: a call the scratch cannot hold fails before any set-up
    const size_t need = sv_workspace_bytes_sample(B, gamma, Vt, Vd, top_p);
    if (need > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_TOO_LARGE;
    if (B == 0 || need == 0)            // nothing to do, or invalid sizes: the checks of the allocating variant
        return spec_verify_sample(target_logits, target_dtype, draft_logits, draft_dtype, draft_tokens, d2t,
                                  u_accept, u_sample, B, gamma, Vt, Vd, temperature, top_p, out_tokens,
                                  out_accept_len, out_p_tok, out_q_tok, out_status, nullptr, 0, stream);
    void *ws = nullptr;
    const sv_status st = scratch_for_current_device(stream, &ws);
    if (st != SV_OK) return st;
    // always the whole array, so the counter region sits at the same place in every call
    return spec_verify_sample(target_logits, target_dtype, draft_logits, draft_dtype, draft_tokens, d2t, u_accept,
                              u_sample, B, gamma, Vt, Vd, temperature, top_p, out_tokens, out_accept_len, out_p_tok,
                              out_q_tok, out_status, ws, SV_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
